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
//     each wave a (BM/2) x (BN/2) tile of MFMA blocks.  The 256 x 256 bf16
//     tiles of the forward products use 8 waves instead (gemm_tile_pp): two
//     per SIMD in two groups that alternate between reading a slice and
//     multiplying it, so one wave's MFMAs cover the other's waits.
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
//   * Remainder tiles: with 256-row tiles, an expert's last <= 64 rows go to
//     a 64-row tile (kRemBM) in the same launch, after all whole tiles (so a
//     split-K tail cuts the small remainder tiles first), and a row count
//     just past a multiple of 256 does not pay for a whole padded tile.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_plan.h"

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
    int rem;                // 1: an expert's last <= kRemThr rows go to kRemBM-row tiles
    int64_t unit_f4;        // float4s of partial accumulators per split unit (main tile)
    int main_blocks;        // blocks [0, main_blocks) take whole tiles, the rest split units
    // k-major B ([K][N] per expert, KM_B launches): row stride of B and the
    // k rows that come from B0 (the rest from B1, row k - K1)
    int64_t ldb;
    int K1;
    // row gather of A (k-contiguous launches): when arows is set, row i of the
    // grouped matrix is row arows[i] / arow_div of A, whose a_bytes bytes the
    // loads may touch (the layer forward reads the activations through the
    // dispatch's assignment ids t k + j in place of a permuted copy)
    const int32_t* arows;
    int64_t a_bytes;
    int arow_div;
};

// Work decomposition.  The plan lists ceil(M_e / BM) row tiles per expert,
// each with NT column tiles, T tiles in all.  When the last round of tiles
// would leave the chip mostly idle (T mod kSplitUnits <= kSplitUnits / 2),
// those `tail` tiles are cut into `split` K ranges each, one block per range:
// every block writes its fp32 partial accumulators, and k_split_fixup adds
// the ranges of a tile in a fixed order and applies the epilogue, so results
// do not depend on timing.  kSplitUnits (tile_plan.h) is the CU count of
// the target chip.

// Remainder tiles.  With 256-row tiles an expert whose row count lies just
// past a multiple of 256 pays a whole tile of padding rows for a few real
// ones.  When at most kRemThr rows are left after an expert's whole tiles,
// they go to ceil(r / kRemBM) tiles of kRemBM rows instead (a quarter of the
// MFMA work of a 256-row tile each), in the same launch, after every whole
// tile.  (Placing them right after their expert's whole tiles of each column
// group, to share the weight panel in L2, measured no faster for the up
// projection and slower for the down projection, whose split-K tail then
// cuts whole tiles instead of remainder tiles.)
#ifndef MOE_GEMM_REM
#define MOE_GEMM_REM 1
#endif
// Schedule of the 256 x 256 bf16 tiles (the forward's up and down
// projections, the backward's products through the weights as stored): 1 =
// gemm_tile_pp, eight waves in two groups that alternate between loading and
// multiplying; 0 = gemm_tile with four waves.  Other tiles always use
// gemm_tile.
#ifndef MOE_GEMM_PP
#define MOE_GEMM_PP 1
#endif
// (kRemBM, kRemThr and whole_tiles: tile_plan.h)

// Tile L of the natural order: first every whole tile, then every remainder
// tile (so that a split-K tail takes remainder tiles first); within each
// kind, experts in order, and inside an expert groups of NG column tiles
// with row tiles fastest inside a group.  The plan holds the whole-tile
// prefix over the experts at [0, E], the remainder-tile prefix at
// [E + 4, 2E + 4].  Returns the expert, the column tile, the first row and
// the row count, and whether it is a remainder tile.
struct TileDesc {
    int e, nt, row0, rows;
    bool rem;
};
__device__ __forceinline__ TileDesc decode_tile(const GemmParams& p, int L, int BM) {
    const int NT = p.NT;
    const int whole_total = p.plan[p.E] * NT;
    TileDesc t;
    t.rem = L >= whole_total;
    const int32_t* pre = t.rem ? p.plan + p.E + 4 : p.plan;
    if (t.rem) L -= whole_total;
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] * NT <= L) lo = mid; else hi = mid;
    }
    t.e = lo;
    const int tiles_e = pre[t.e + 1] - pre[t.e];
    const int local = L - pre[t.e] * NT;
    constexpr int NG = 8;
    const int grp = local / (tiles_e * NG);
    const int inside = local - grp * tiles_e * NG;
    const int mt = inside % tiles_e;
    t.nt = grp * NG + inside / tiles_e;
    const int off = p.offsets[t.e], M = p.offsets[t.e + 1] - off;
    if (t.rem) {
        t.row0 = off + whole_tiles(M, BM, true) * BM + mt * kRemBM;
        t.rows = min(kRemBM, off + M - t.row0);
    } else {
        t.row0 = off + mt * BM;
        t.rows = min(BM, off + M - t.row0);
    }
    return t;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row.  LDS serves
// 16 lanes of a 16-byte read per pass: rows r .. r+15 at one logical chunk
// then cover every (row parity, physical chunk) pair, i.e. 16 distinct
// 16-byte bank groups.  Depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Operand layouts of gemm_tile: both k-contiguous (the forward products), or
// B k-major (B_e stored [K][N]: the backward's products through a weight as
// stored, dh = dy W2 and dx = [da | du] [W1; W3]).
enum { KM_NONE = 0, KM_B = 1 };

// A k-major B slice is 64 k rows of the tile's BN columns (2 BN bytes per
// row, the same 32 KB as 256 rows of 128 bytes at BN = 256).  Fragments come
// from ds_read_b64_tr_b16: within 16 lanes, lane L reads 8 bytes (4 columns)
// of k row L / 4 and receives column L of 4 k rows, so two reads give a lane
// the 8 consecutive k of one column that an MFMA operand holds.  The 16-byte
// chunks of a row are XOR swizzled by swzk(k row) in bits 1..3: the 8 k rows
// that 32 lanes read in one pass (4 rows of each of two lane groups) then
// fall in 8 distinct 32-byte bank groups.  Needs BN >= 128 (16 chunks per
// row).
__device__ __forceinline__ int swzk(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 1; }

// Direct-to-LDS 16-byte buffer load issued as an instruction the compiler does
// not model.  Launches that read LDS with ds_read_b64_tr_b16 use it for every
// slice load: for a load it issues itself the compiler cannot tell which LDS
// bytes it writes and waits for all of them before every transposing read,
// which would drain the ring.  Ordering comes from the explicit vmcnt waits
// and barriers of the pipeline; the instruction writes no register.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, const lds_u8* dst) {
    const uint32_t m0 = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(m0), "s"(soff)
                 : "memory");
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;

// Ring depths of the A and B slices.  Batch j (issued after the barrier of
// slice j) loads A slice j + NA and B slice j + NB, in that order; before that
// barrier a wave waits until slice j + 1 has landed, which leaves `wait`
// of its own loads in flight (`wait0` before the first slice).  NB is NA or
// NA + 1; the depths maximise `wait` within 160 KB of LDS.
struct RingDepth {
    int na, nb, wait, wait0, bytes;
};
constexpr RingDepth ring_depth(int BM, int BN, int NW) {
    const int SA = BM * 128, SB = BN * 128, ga = BM / 8 / NW, gb = BN / 8 / NW;
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
// MFMA block edge of the bf16 products: 32 (v_mfma_f32_32x32x16_bf16) or
// 16 (v_mfma_f32_16x16x32_bf16); fp32 always uses 16x16x4 blocks.
#ifndef MOE_GEMM_MB_BF16
#define MOE_GEMM_MB_BF16 16
#endif
template <bool BF16>
constexpr int mfma_block() { return BF16 ? MOE_GEMM_MB_BF16 : 16; }

template <bool BF16, int BM, int BN, int EPI, int WGM, int WGN>
struct GemmEpilogue {
    static constexpr int NW = WGM * WGN;       // waves: WGM along M, WGN along N
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int MB = mfma_block<BF16>();
    static constexpr int FM = WM / MB, FN = WN / MB;
    static constexpr int RA = MB == 32 ? 16 : 4;   // accumulator registers per MFMA block
    typedef typename std::conditional<MB == 32, floatx16_t, floatx4_t>::type acc_t;

    // A lane's accumulators are RA / 4 groups of 4 consecutive output columns
    // of one token row.  16x16 block: lane l, element t holds D[n = 4(l/16) +
    // t][m = l % 16]; 32x32 block: element 4g + t holds D[n = 8g + 4(l/32) +
    // t][m = l % 32].  Column offset of group g inside the block:
    __device__ static int group_col(int g, int lane) { return MB == 32 ? 8 * g + 4 * (lane >> 5) : 4 * (lane >> 4); }

    // float4 index of partial element (i, j, 4*r4 .. 4*r4+3) of wave w, unit
    // u (units are p.unit_f4 float4s apart whatever the tile's row count)
    __device__ static int64_t partial_index(const GemmParams& p, int u, int w, int i, int j, int r4, int lane) {
        return (int64_t)u * p.unit_f4 + ((((int64_t)w * FN + i) * FM + j) * (RA / 4) + r4) * 64 + lane;
    }

    __device__ static void store_partial(const GemmParams& p, const acc_t (&acc)[FN][FM], int u, int w, int lane) {
        float4* dst = (float4*)p.partial;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r4 = 0; r4 < RA / 4; ++r4)
                    dst[partial_index(p, u, w, i, j, r4, lane)] =
                        make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
    }

    // Column groups of the epilogue: the MB-row blocks i of the wave's B tile
    // are independent, except that SwiGLU pairs block 2p (gate) with block
    // 2p+1 (up).
    static constexpr int IG = epi_swiglu(EPI) ? 2 : 1;

    // Output of blocks i0 .. i0+IG-1 (acc[0 .. IG-1]): a lane stores each of
    // its groups of 4 consecutive output columns at once.
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
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = wm * WM + j * MB + (lane & (MB - 1));
            if (m >= rows) continue;
#pragma unroll
            for (int g = 0; g < RA / 4; ++g) {
                if constexpr (epi_swiglu(EPI)) {
                    const int fblock = (wn * FN + i0) >> 1;        // MB-row blocks alternate gate / up
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = silu_mul(acc[0][j][4 * g + t], acc[1][j][4 * g + t]);
                    const int64_t col = (int64_t)nt * (BN / 2) + fblock * MB + group_col(g, lane);
                    store4(m, col, v);
                    if constexpr (epi_save(EPI)) {
                        float a[4], u[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            a[t] = acc[0][j][4 * g + t];
                            u[t] = acc[1][j][4 * g + t];
                        }
                        store4_to(p.C2, p.ldc2, m, col, a);
                        store4_to(p.C2, p.ldc2, m, p.N + col, u);
                    }
                } else {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float x = acc[0][j][4 * g + t];
                        if constexpr (epi_relu(EPI)) x = fmaxf(x, 0.0f);
                        v[t] = x;
                    }
                    const int64_t col = (int64_t)nt * BN + wn * WN + i0 * MB + group_col(g, lane);
                    store4(m, col, v);
                    if constexpr (epi_save(EPI)) {
                        float a[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) a[t] = acc[0][j][4 * g + t];
                        store4_to(p.C2, p.ldc2, m, col, a);
                    }
                }
            }
        }
    }

    // bf16 output through LDS (plain, ReLU and SwiGLU epilogues, 16x16
    // blocks): a wave writes its outputs to its own LDS region, rows padded by
    // 16 bytes (the 16 rows x 2 column groups of a half wave then hit 32
    // distinct bank pairs), and stores whole rows back, 16 bytes per lane, so
    // every global write covers whole 128-byte lines.  The direct form writes
    // 32 bytes of each of 16 rows per instruction: partial lines, which cost
    // the down projection about 14 % of its time.
    static constexpr int OC = epi_swiglu(EPI) ? WN / 2 : WN;   // output columns per wave
    static constexpr int PITCH = OC * 2 + 16;                  // LDS bytes per staged row
    static constexpr int STAGE_BYTES = NW * WM * PITCH;
    static constexpr bool can_stage = BF16 && MB == 16 && !epi_save(EPI) && (OC * 2) % 16 == 0 && 64 % (OC * 2 / 16) == 0;
    __device__ static void store_staged(const GemmParams& p, const acc_t (&acc)[FN][FM], int row0, int rows, int nt,
                                        int wm, int wn, int lane, int wave, lds_u8* lds) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) u32x2_t lds_u2;
        typedef __attribute__((address_space(3))) u32x4_t lds_u4;
        lds_u8* reg = lds + wave * WM * PITCH;
        auto silu_mul = [](float gt, float up) { return gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up; };
#pragma unroll
        for (int i0 = 0; i0 < FN; i0 += IG) {
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = j * MB + (lane & (MB - 1));
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if constexpr (epi_swiglu(EPI)) {
                        v[t] = silu_mul(acc[i0][j][t], acc[i0 + 1][j][t]);
                    } else {
                        float x = acc[i0][j][t];
                        if constexpr (epi_relu(EPI)) x = fmaxf(x, 0.0f);
                        v[t] = x;
                    }
                }
                const int cl = (epi_swiglu(EPI) ? (i0 >> 1) : i0) * MB + group_col(0, lane);
                u32x2_t w;
                w[0] = pack_bf16x2(v[0], v[1]);
                w[1] = pack_bf16x2(v[2], v[3]);
                *(lds_u2*)(reg + m * PITCH + cl * 2) = w;
            }
        }
        // the region is this wave's own and its LDS accesses complete in order
        constexpr int LPR = OC * 2 / 16, RPI = 64 / LPR;          // lanes per row, rows per instruction
        const int lr = lane / LPR, lc = lane % LPR;
        const int64_t col0 = epi_swiglu(EPI) ? (int64_t)nt * (BN / 2) + wn * OC : (int64_t)nt * BN + wn * WN;
#pragma unroll
        for (int r = 0; r < WM; r += RPI) {
            const int m = r + lr;
            const u32x4_t v = *(lds_u4*)(reg + m * PITCH + lc * 16);
            const int grow = wm * WM + m;
            if (grow < rows) *(u32x4_t*)((uint16_t*)p.C + (int64_t)(row0 + grow) * p.ldc + col0 + lc * 8) = v;
        }
    }

    __device__ static void store(const GemmParams& p, const acc_t (&acc)[FN][FM], int row0, int rows, int nt, int wm,
                                 int wn, int lane) {
#pragma unroll
        for (int i0 = 0; i0 < FN; i0 += IG) store_cols(p, acc + i0, i0, row0, rows, nt, wm, wn, lane);
    }
};

// One tile of the grouped GEMM (rows [t.row0, t.row0 + t.rows) of expert
// t.e, column tile t.nt, K slices [k0, k1)); `lds` is the kernel's LDS.
// unit >= 0: a split unit, which stores its fp32 partial accumulators.
// KM: operand layout (KM_NONE or KM_B; see swzk).  STG: the output goes
// through LDS (epilogues that can stage, and C / ldc aligned for it, checked
// by the host); the direct-store form is a separate instantiation because
// compiled into the same kernel it raises the register demand past the file
// and the compiler spills accumulators around the epilogue.
template <bool BF16, int BM, int BN, int EPI, int WGN, int KM = KM_NONE, bool STG = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, lds_u8* lds, const TileDesc& t, int k0, int k1,
                                          int unit) {
    constexpr int NW = 2 * WGN;               // waves: 2 along M, WGN along N
    constexpr int WM = BM / 2, WN = BN / WGN;
    constexpr int MB = mfma_block<BF16>();    // MFMA block edge (32x32x16 or 16x16x32 bf16, 16x16x4 fp32)
    constexpr int FM = WM / MB, FN = WN / MB;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int KS = MB == 32 ? 2 : 1;      // k-steps per half slice (64 bytes of K)
    constexpr int SA = BM * 128, SB = BN * 128;
    constexpr RingDepth RD = ring_depth(BM, BN, NW);
    constexpr int NA = RD.na, NB = RD.nb;
    constexpr int GA = BM / 8, GB = BN / 8;   // 1 KB load groups: 8 rows x 128 bytes
    constexpr int ga = GA / NW, gb = GB / NW; // groups per wave
    static_assert(GA % NW == 0 && GB % NW == 0, "load groups split evenly over the waves");
    typedef GemmEpilogue<BF16, BM, BN, EPI, 2, WGN> Epi;
    typedef typename Epi::acc_t acc_t;
    static_assert(FM >= 1 && FN >= 1, "tile smaller than one MFMA block");
    static_assert(!epi_swiglu(EPI) || (FN % 2) == 0, "SwiGLU pairs MB-row blocks");
    static_assert(RD.wait0 < 64 && RD.bytes <= 160 * 1024, "ring exceeds vmcnt or LDS");
    typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
    const int e = t.e, nt = t.nt, row0 = t.row0, rows = t.rows;
    constexpr bool BKM = KM == KM_B;
    static_assert(KM == KM_NONE || (BF16 && EPI == EPI_STORE && MB == 16 && BN >= 128),
                  "k-major B: bf16, plain store, 16x16 blocks, k rows of at least 256 bytes");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- direct-to-LDS loads.  Slot layout: NA A slots of BM rows, then NB B
    // slots of BN rows, 128 bytes per row.  One buffer_load_dwordx4 ... lds of
    // a wave fills a 1 KB group: lane l lands at byte 16*l, i.e. row
    // 8*g + l/8, physical chunk l%8, and fetches logical chunk (l%8) ^ swz(row)
    // (the swizzle is applied on the global side).  Each wave loads ga A
    // groups and gb B groups of every slice.  Addresses are buffer descriptors
    // (SGPRs) holding the tile's base and extent, a 32-bit lane offset, and
    // the K offset in an SGPR.
    constexpr int kRsrcWord3 = 0x00020000;
    __amdgpu_buffer_rsrc_t rsA, rsB0, rsB1;
    uint32_t voffA[ga], voffB[gb];
    if (KM == KM_NONE && p.arows) {
        rsA = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, (int)p.a_bytes, kRsrcWord3);
#pragma unroll
        for (int q = 0; q < ga; ++q) {
            const int r = 8 * (wave * ga + q) + (lane >> 3);
            voffA[q] = (uint32_t)(p.arows[row0 + min(r, rows - 1)] / p.arow_div) * (uint32_t)(p.lda * ES) +
                       (uint32_t)(((lane & 7) ^ swz(r)) << 4);
        }
    } else {
        rsA = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.A + (int64_t)row0 * p.lda * ES), (short)0,
                                                (int)(((int64_t)(rows - 1) * p.lda + p.K) * ES), kRsrcWord3);
#pragma unroll
        for (int q = 0; q < ga; ++q) {
            const int r = 8 * (wave * ga + q) + (lane >> 3);
            voffA[q] = (uint32_t)(min(r, rows - 1) * (int)p.lda * ES + (((lane & 7) ^ swz(r)) << 4));
        }
    }
    if constexpr (BKM) {
        // B_e stored [K][N]: k rows below K1 from B0, the rest from B1.  A
        // 1 KB load group is 512 / BN k rows of the tile's BN columns: lane l
        // takes k row g (512 / BN) + l / (BN / 8), physical chunk l % (BN / 8),
        // and fetches logical chunk (l % (BN / 8)) ^ swzk(k row)
        const int64_t boff = (int64_t)e * p.bstride * ES;
        rsB0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.B0 + boff), (short)0,
                                                 (int)((int64_t)p.K1 * p.ldb * ES), kRsrcWord3);
        rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)(p.B1 ? p.B1 : p.B0) + boff), (short)0,
                                                 (int)((int64_t)(p.K - p.K1) * p.ldb * ES), kRsrcWord3);
#pragma unroll
        for (int q = 0; q < gb; ++q) {
            const int kr = (wave * gb + q) * (512 / BN) + lane / (BN / 8);
            const int c = (lane % (BN / 8)) ^ swzk(kr);
            voffB[q] = (uint32_t)(((int64_t)kr * p.ldb + nt * BN + 8 * c) * ES);
        }
    } else {
        const int64_t brow_base = epi_swiglu(EPI) ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;
        const int b_rows = epi_swiglu(EPI) ? BN / 2 : BN;
        const int64_t boff = ((int64_t)e * p.bstride + brow_base * p.K) * ES;
        rsB0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.B0 + boff), (short)0,
                                                 (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
        rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)(epi_swiglu(EPI) ? p.B1 : p.B0) + boff),
                                                 (short)0, (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
#pragma unroll
        for (int q = 0; q < gb; ++q) {
            const int g = wave * gb + q;
            const int r = 8 * g + (lane >> 3);
            // SwiGLU: MB-row block j of the tile is rows (j/2)*MB .. +MB-1 of W1
            // (j even) or W3 (j odd); a group is 8 rows, so block j = g / (MB/8)
            const int rr = epi_swiglu(EPI) ? ((g / (MB / 4)) * MB + (r & (MB - 1))) : r;
            voffB[q] = (uint32_t)(rr * p.K * ES + (((lane & 7) ^ swz(r)) << 4));
        }
    }
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const int nk = k1 - k0;
    // virtual slice v goes to slot v % N; slices past the end reload the last
    // one into a free slot (nobody reads it), which keeps the per-wave load
    // count of every batch the same
    auto issueA1 = [&](int v, int q) {      // group q of this wave's part of A slice v
        lds_u8* dst = &lds[(v % NA) * SA + wave * ga * 1024];
        const int kk = k0 + min(v, nk - 1);
        if constexpr (KM == KM_NONE) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)(dst + q * 1024), 16, voffA[q], kk * 128, 0, 0);
        } else {
            dma16(rsA, voffA[q], (uint32_t)(kk * 128), dst + q * 1024);
        }
    };
    auto issueB1 = [&](int v, int q) {
        lds_u8* dst = &lds[NA * SA + (v % NB) * SB + wave * gb * 1024];
        const int kk = k0 + min(v, nk - 1);
        if constexpr (KM == KM_NONE) {
            const bool up = epi_swiglu(EPI) && (((wave * gb + q) / (MB / 8)) & 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(up ? rsB1 : rsB0, (lds_ptr_t)(dst + q * 1024), 16, voffB[q],
                                                     kk * 128, 0, 0);
        } else {
            const int kr = kk * 64;
            const bool hi = kr >= p.K1;
            dma16(hi ? rsB1 : rsB0, voffB[q], (uint32_t)((int64_t)(hi ? kr - p.K1 : kr) * p.ldb * ES),
                  dst + q * 1024);
        }
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
            for (int r = 0; r < Epi::RA; ++r) acc[i][j][r] = 0.0f;

    // Fragment reads, per half slice h (64 bytes of K, 4 chunks of 16
    // bytes): 16x16 blocks: lane l takes row l % 16 at logical chunk
    // 4h + l/16 (8 bf16 k values, one 16x16x32 MFMA; or 4 fp32 k values,
    // four 16x16x4 MFMAs); 32x32 blocks: k-step s2 (2 chunks) of the half,
    // lane l takes row l % 32 at chunk 4h + 2 s2 + l/32 (8 bf16 k values of
    // one 32x32x16 MFMA).  Weights are MFMA source 0 (rows = output columns
    // n), activations source 1 (columns = token rows m).  The swizzle depends
    // on the row mod 16 only, so blocks i of one operand differ by the
    // constant i*MB*128.
    constexpr int NF = KS * (FM + FN);       // fragments per half slice
    int fo[2][KS][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const int lr = lane & (MB - 1);
            const int ch = MB == 32 ? 4 * h + 2 * s2 + (lane >> 5) : 4 * h + (lane >> 4);
            fo[h][s2][0] = (wm * WM + lr) * 128 + ((ch ^ swz(lr)) << 4);
            fo[h][s2][1] = NA * SA + (wn * WN + lr) * 128 + ((ch ^ swz(lr)) << 4);
        }
    // fragment r of half slice h: k-step r / (FM + FN), then FM A blocks and
    // FN B blocks
    // k-major B: lane base address of each MFMA block of the wave (k rows
    // 8 (l/16) + (l%16)/4 of the slice, 4 columns at (l%4) * 4 of the block);
    // half h adds 32 k rows, the second read of a fragment 4 more.  Within a
    // slice the swizzle of these rows is the lane constant sw.
    constexpr int RBB = BN * 2;
    int kbb[BKM ? FN : 1];
    if constexpr (BKM) {
        const int g4 = lane >> 4, L = lane & 15;
        const int sw = ((L >> 2) | ((g4 & 1) << 2)) << 1;
        const int kr = 8 * g4 + (L >> 2);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int col = wn * WN + i * 16 + 4 * (L & 3);
            kbb[i] = NA * SA + kr * RBB + (((col >> 3) ^ sw) << 4) + ((col & 7) << 1);
        }
    }
    auto trfrag = [&](int off, int rowbytes) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off + 4 * rowbytes));
        typedef short v8i16_t __attribute__((ext_vector_type(8)));
        const v8i16_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(u32x4_t, both);
    };
    auto read1 = [&](int ks, int h, u32x4_t* f, int r) {
        const int s2 = r / (FM + FN), q = r % (FM + FN);
        if (q < FM) {
            f[r] = *(lds_u32x4*)(&lds[(ks % NA) * SA] + fo[h][s2][0] + q * MB * 128);
        } else {
            if constexpr (BKM) f[r] = trfrag((ks % NB) * SB + kbb[q - FM] + 32 * h * RBB, RBB);
            else f[r] = *(lds_u32x4*)(&lds[(ks % NB) * SB] + fo[h][s2][1] + (q - FM) * MB * 128);
        }
    };
    // one bf16 MFMA of the block shape: acc += W-fragment x activation-fragment
    auto mfma_bf16 = [](const u32x4_t& fw, const u32x4_t& fx, acc_t& a) {
        if constexpr (MB == 32)
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fw),
                                                        __builtin_bit_cast(bf16x8_t, fx), a, 0, 0, 0);
        else
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fw),
                                                        __builtin_bit_cast(bf16x8_t, fx), a, 0, 0, 0);
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
                        mfma_bf16(fb, fa, acc[i][j]);
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
            mfma_bf16(f[s2 * (FM + FN) + FM + i], f[s2 * (FM + FN) + j], acc[i][j]);
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
    // the first half, B in the second) are dealt evenly over the chunks, and
    // the fragment reads of the other set go into the first CH/2 chunks, so they
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
        // chunks per half region: 32 of 2 MFMAs at the 256 x 256 tile (1.2 %
        // faster than 8 chunks of 8 on the Mixtral up GEMM, the loads and the
        // fragment reads then sit between smaller MFMA groups)
        constexpr int CH = NMMA < 32 ? NMMA : 32;
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

    if (unit >= 0) {
        Epi::store_partial(p, acc, unit, wave, lane);
    } else if constexpr (Epi::can_stage && STG) {
        static_assert(Epi::STAGE_BYTES <= RD.bytes, "staged output fits in the ring's LDS");
        // every wave is past its last fragment read and its slice loads have
        // landed: the ring's LDS is free for the staged output
        lds_barrier();
        Epi::store_staged(p, acc, row0, rows, nt, wm, wn, lane, wave, lds);
    } else {
        Epi::store(p, acc, row0, rows, nt, wm, wn, lane);
    }
}

// Ping-pong schedule of the 256 x 256 bf16 tile with k-contiguous operands.
// Eight waves, two per SIMD (waves w and w + 4 share one).  Group G = wave / 4
// computes rows [128 G, 128 G + 128) of the tile and wave q = wave % 4 of the
// group the columns [64 q, 64 q + 64) (wm = G, wn = q of the 2 x 4 epilogue
// layout).  Each group alternates between a memory phase (read the current
// slice's 24 fragments into registers) and a compute phase (the slice's 64
// MFMAs on registers only), with a block barrier between phases and group 1
// one phase behind group 0: on every SIMD one wave multiplies while the other
// waits on LDS, memory or the barrier, so the matrix unit does not idle
// while a wave stalls.
//   barriers 2k .. 2k+1:   group 0 memory phase of slice k, group 1 compute k-1
//   barriers 2k+1 .. 2k+2: group 0 compute k, group 1 memory phase of slice k
// Slice s must be in LDS at barrier 2s.  Group 0 loads all of A into a ring
// of 2 slots, group 1 all of B into a ring of 3 (5 slots of 32 KB in all).
// The slot of slice s is free once group 1's memory phase of s has ended
// (barrier 2s + 2).  Each group issues its slice k - 1 + N (N its ring's
// slots) in its memory phase of slice k, into the slot of slice k - 1: A
// slice k + 1 then has 2 phases to land, B slice k + 2 has 3, and every
// phase carries the loads of one operand (issuing group 1's loads a phase
// earlier puts both operands' loads into one phase, and that burst stalls
// the address unit: measured 16 % slower).  Before barrier 2k + 2 a wave
// waits for its own loads of slice k + 1.  Both groups pass 2 nk + 1
// barriers and no load goes past the last slice; after the last barrier
// every LDS read and load is complete, so the epilogue stages through the
// ring's LDS without a further barrier.
// With KM == KM_B (B_e stored [K][N], see swzk) the B slices are 64 k rows of
// the tile's 256 columns, their fragments come from transposing reads, and
// every slice load is a dma16 (see there).
template <int EPI, bool STG, int KM = KM_NONE>
__device__ __forceinline__ void gemm_tile_pp(const GemmParams& p, lds_u8* lds, const TileDesc& t, int k0, int k1,
                                             int unit) {
    constexpr int BM = 256, BN = 256, WGN = 4, MB = 16;
    constexpr int WM = BM / 2, WN = BN / WGN, FM = WM / MB, FN = WN / MB;   // 128 x 64 per wave: 8 x 4 blocks
    constexpr int SL = 256 * 128;                                          // bytes of an A or a B slice
    constexpr int NA = 2, NB = 3;
    constexpr int GL = 8;            // 1 KB load groups per wave and slice (32 per operand, 4 waves)
    constexpr int NF = FM + FN;      // fragments per half slice
    constexpr int ES = 2;
    typedef GemmEpilogue<true, BM, BN, EPI, 2, WGN> Epi;
    typedef typename Epi::acc_t acc_t;
    static_assert((NA + NB) * SL <= 160 * 1024, "rings fit in LDS");
    static_assert(!epi_swiglu(EPI) || (FN % 2) == 0, "SwiGLU pairs MB-row blocks");
    constexpr bool BKM = KM == KM_B;
    static_assert(!BKM || EPI == EPI_STORE, "k-major B: plain store");
    typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const int e = t.e, nt = t.nt, row0 = t.row0, rows = t.rows;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = wave >> 2, q = wave & 3;
    const int nk = k1 - k0;
    constexpr int kRsrcWord3 = 0x00020000;

    // Slice loads (as in gemm_tile): group 0 wave q fills A rows
    // [64 q, 64 q + 64) of a slot, group 1 wave q B rows [64 q, 64 q + 64);
    // load group g of the wave is slot rows 8 (8 q + g) .. + 7.
    __amdgpu_buffer_rsrc_t rs0, rs1;
    // lane offsets of the loads; the k-major launches keep three lane
    // constants instead and form each offset when the load is issued (eight
    // offsets in registers made the compiler spill them inside the loop)
    uint32_t voff[BKM ? 1 : GL];
    uint32_t lc0 = 0, lc1 = 0, lc2 = 0;
    if (G == 0 && !BKM && p.arows) {
        // gathered rows: the descriptor spans A, each lane its row's offset
        rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, (int)p.a_bytes, kRsrcWord3);
        rs1 = rs0;
#pragma unroll
        for (int g = 0; g < GL; ++g) {
            const int r = 8 * (8 * q + g) + (lane >> 3);
            voff[g] = (uint32_t)(p.arows[row0 + min(r, rows - 1)] / p.arow_div) * (uint32_t)(p.lda * ES) +
                      (uint32_t)(((lane & 7) ^ swz(r)) << 4);
        }
    } else if (G == 0) {
        rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.A + (int64_t)row0 * p.lda * ES), (short)0,
                                                (int)(((int64_t)(rows - 1) * p.lda + p.K) * ES), kRsrcWord3);
        rs1 = rs0;
        if constexpr (BKM) {
            lc0 = (uint32_t)(64 * q + (lane >> 3));                      // A row of load group 0
            lc1 = (uint32_t)(((lane & 7) ^ (lane >> 4)) << 4);            // chunk offset, even groups
            lc2 = (uint32_t)(((lane & 7) ^ (4 + (lane >> 4))) << 4);      // chunk offset, odd groups
        } else {
#pragma unroll
            for (int g = 0; g < GL; ++g) {
                const int r = 8 * (8 * q + g) + (lane >> 3);
                voff[g] = (uint32_t)(min(r, rows - 1) * (int)p.lda * ES + (((lane & 7) ^ swz(r)) << 4));
            }
        }
    } else if constexpr (BKM) {
        // k rows below K1 from B0, the rest from B1; load group gg = 8 q + g
        // is k rows 2 gg, 2 gg + 1 of the slice: lane l takes k row
        // 2 gg + l / 32, physical chunk l % 32, logical chunk (l % 32) ^ swzk
        const int64_t boff = (int64_t)e * p.bstride * ES;
        rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.B0 + boff), (short)0,
                                                (int)((int64_t)p.K1 * p.ldb * ES), kRsrcWord3);
        rs1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)(p.B1 ? p.B1 : p.B0) + boff), (short)0,
                                                (int)((int64_t)(p.K - p.K1) * p.ldb * ES), kRsrcWord3);
        lc0 = (uint32_t)(((int64_t)(16 * q + (lane >> 5)) * p.ldb + nt * BN) * ES);   // k row of load group 0
        lc1 = (uint32_t)((lane & 31) ^ ((lane >> 5) << 1));                           // chunk before swzk's g bits
    } else {
        const int64_t brow_base = epi_swiglu(EPI) ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;
        const int b_rows = epi_swiglu(EPI) ? BN / 2 : BN;
        const int64_t boff = ((int64_t)e * p.bstride + brow_base * p.K) * ES;
        rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.B0 + boff), (short)0,
                                                (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
        rs1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)(epi_swiglu(EPI) ? p.B1 : p.B0) + boff),
                                                (short)0, (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
#pragma unroll
        for (int g = 0; g < GL; ++g) {
            const int gg = 8 * q + g;
            const int r = 8 * gg + (lane >> 3);
            // SwiGLU: 16-row block j = gg / 2 of the tile is rows (j / 2) 16 ..
            // + 15 of W1 (j even) or W3 (j odd)
            const int rr = epi_swiglu(EPI) ? ((gg / 4) * MB + (r & (MB - 1))) : r;
            voff[g] = (uint32_t)(rr * p.K * ES + (((lane & 7) ^ swz(r)) << 4));
        }
    }
    const int N = G == 0 ? NA : NB;                  // slots of this wave's ring
    lds_u8* const ring = &lds[G == 0 ? 0 : NA * SL];
    // this wave's share of slice v of its operand, if v is a slice of the range
    auto issue = [&](int v) {
        if (v >= nk) return;
        const int kk = k0 + v;
        lds_u8* dst = ring + (v % N) * SL + q * GL * 1024;
        if constexpr (BKM) {
            if (G == 0) {
                // A row 64 q + 8 g + l / 8 (clamped to the tile's last row),
                // chunk (l % 8) ^ swz(row) with swz(row) = 4 (g % 2) + l / 16
#pragma unroll
                for (int g = 0; g < GL; ++g) {
                    const uint32_t r = min(lc0 + 8 * g, (uint32_t)(rows - 1));
                    dma16(rs0, r * (uint32_t)(p.lda * ES) + ((g & 1) ? lc2 : lc1), (uint32_t)(kk * 128), dst + g * 1024);
                }
            } else {
                // k row 16 q + 2 g + l / 32 of the slice; its swzk is
                // 2 (l / 32) + 4 (g % 2) + 8 (g / 4), whose g bits are a constant
                const int kr = kk * 64;
                const bool hi = kr >= p.K1;
                const __amdgpu_buffer_rsrc_t rs = hi ? rs1 : rs0;
                const uint32_t soff = (uint32_t)((int64_t)(hi ? kr - p.K1 : kr) * p.ldb * ES);
#pragma unroll
                for (int g = 0; g < GL; ++g) {
                    const uint32_t c = lc1 ^ (uint32_t)((4 * (g & 1) + 8 * (g >> 2)));
                    dma16(rs, lc0 + (uint32_t)(2 * g * p.ldb * ES) + c * 16, soff, dst + g * 1024);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < GL; ++g) {
                // SwiGLU B: gate rows for (g / 2) even, up rows for odd (8 q is even)
                const bool up = G != 0 && epi_swiglu(EPI) && ((g >> 1) & 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(up ? rs1 : rs0, (lds_ptr_t)(dst + g * 1024), 16, voff[g],
                                                         kk * 128, 0, 0);
            }
        }
    };
    // before barrier 2k + 2: this wave's loads of slice k + 1 have landed
    // (with a ring of 3 the next slice's loads may stay in flight)
    auto wait_next = [&](int k) {
        if (N == 3 && k + 2 < nk) wait_vmcnt<GL>();
        else wait_vmcnt<0>();
    };

    // Fragments of slice s (both halves): lane l reads row l % 16 of each
    // 16-row block at logical chunk 4 h + l / 16.
    int foA[2], foB[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int lr = lane & (MB - 1), ch = 4 * h + (lane >> 4);
        foA[h] = (G * WM + lr) * 128 + ((ch ^ swz(lr)) << 4);
        foB[h] = NA * SL + (q * WN + lr) * 128 + ((ch ^ swz(lr)) << 4);
    }
    // k-major B: lane base of each 16-column block of the wave (k rows
    // 8 (l / 16) + (l % 16) / 4 of the slice, 4 columns at 4 (l % 4)); half h
    // adds 32 k rows, a fragment's second read 4 more (as in gemm_tile)
    constexpr int RBB = BN * 2;
    int kbb[BKM ? FN : 1];
    if constexpr (BKM) {
        const int g4 = lane >> 4, L = lane & 15;
        const int sw = ((L >> 2) | ((g4 & 1) << 2)) << 1;
        const int kr = 8 * g4 + (L >> 2);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int col = q * WN + i * 16 + 4 * (L & 3);
            kbb[i] = NA * SL + kr * RBB + (((col >> 3) ^ sw) << 4) + ((col & 7) << 1);
        }
    }
    u32x4_t f[2 * NF];
    auto read_slice = [&](int s) {
        const lds_u8* a = &lds[(s % NA) * SL];
        const lds_u8* b = &lds[(s % NB) * SL];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < FM; ++j) f[h * NF + j] = *(lds_u32x4*)(a + foA[h] + j * MB * 128);
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                if constexpr (BKM) {
                    const lds_u8* bp = b + kbb[i] + 32 * h * RBB;
                    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)bp);
                    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(bp + 4 * RBB));
                    typedef short v8i16_t __attribute__((ext_vector_type(8)));
                    const v8i16_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    f[h * NF + FM + i] = __builtin_bit_cast(u32x4_t, both);
                } else {
                    f[h * NF + FM + i] = *(lds_u32x4*)(b + foB[h] + i * MB * 128);
                }
            }
        }
    };
    acc_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // the slice's MFMAs at raised issue priority, so the SIMD's other wave
    // (in its memory phase) takes only the issue slots they leave
    auto compute = [&]() {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f[h * NF + FM + i]),
                                                                        __builtin_bit_cast(bf16x8_t, f[h * NF + j]),
                                                                        acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };
    // phase boundary: nothing moves across it
    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // memory phase of slice k: the fragments of slice k, then this wave's
    // loads of slice k - 1 + N (into the slot of slice k - 1).  The reads
    // go first so they are not queued behind the slice loads' LDS writes:
    // up GEMM 1468 -> 1414 us against loads first (Mixtral, same box,
    // bit-identical); dealing the loads out between the reads measured level.
    auto memory = [&](int k) {
        read_slice(k);
        issue(k - 1 + N);
    };

    // prologue: slices 0 .. N - 2 of the ring, slice 0 landed
    issue(0);
    if (N == 3) issue(1);
    wait_next(-1);
    phase_barrier();                             // barrier 0
    if (G == 0) {
        for (int k = 0; k < nk; ++k) {
            memory(k);
            phase_barrier();                     // barrier 2k + 1
            compute();
            wait_next(k);
            phase_barrier();                     // barrier 2k + 2
        }
    } else {
        phase_barrier();                         // barrier 1
        for (int k = 0; k < nk; ++k) {
            memory(k);
            wait_next(k);
            phase_barrier();                     // barrier 2k + 2
            compute();
            if (k + 1 < nk) phase_barrier();     // barrier 2k + 3
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    if (unit >= 0) {
        Epi::store_partial(p, acc, unit, wave, lane);
    } else if constexpr (Epi::can_stage && STG) {
        static_assert(Epi::STAGE_BYTES <= (NA + NB) * SL, "staged output fits in the ring's LDS");
        Epi::store_staged(p, acc, row0, rows, nt, G, q, lane, wave, lds);
    } else {
        Epi::store(p, acc, row0, rows, nt, G, q, lane);
    }
}

// LDS bytes of a launch: its tile's ring, or the larger of that and the
// remainder tile's ring when remainder tiles can occur (256-row bf16 tiles).
template <bool BF16, int BM, int BN, int WGN>
constexpr int gemm_lds_bytes() {
    constexpr int main_bytes = ring_depth(BM, BN, 2 * WGN).bytes;
    if constexpr (BF16 && BM == 256) {
        constexpr int rem_bytes = ring_depth(kRemBM, BN, 2 * WGN).bytes;
        return main_bytes > rem_bytes ? main_bytes : rem_bytes;
    }
    return main_bytes;
}

// The grouped GEMM kernel: finds its work unit and runs its tile.  Blocks
// [0, p.main_blocks) take whole tiles: block ids are dealt round-robin to the
// 8 XCDs, so tiles are remapped to give each XCD a contiguous range (its
// blocks share weight and activation panels in its L2).  Later blocks are the
// split-K units of the tail: block p.main_blocks + u is unit u, range
// u % split of tail tile u / split; being dispatched last, they fill the CUs
// that the last round of whole tiles leaves idle.  Remainder tiles
// (256-row bf16 launches) run with 64-row tiles; whole 256 x 256 tiles with
// the ping-pong schedule.
template <bool BF16, int BM, int BN, int EPI, int WGN, int KM = KM_NONE, bool STG = false>
__global__ __launch_bounds__(128 * WGN) void k_grouped_gemm(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    __shared__ __align__(16) uint8_t lds_mem[gemm_lds_bytes<BF16, BM, BN, WGN>()];
    lds_u8* lds = (lds_u8*)lds_mem;
    const int total = (p.plan[p.E] + p.plan[2 * p.E + 4]) * p.NT;
    const int full = p.plan[p.E + 1], split = p.plan[p.E + 2], tail = p.plan[p.E + 3];
    int L, k0 = 0, k1 = p.nk, unit = -1;
    if ((int)blockIdx.x < p.main_blocks) {
        // The tiles run as whole units (all but a split tail) are nw whole and
        // nr remainder tiles; XCD x takes an equal share of each, as
        // contiguous ranges, and deals its remainder tiles evenly among its
        // whole tiles: the remainder tiles reread their experts' weights from
        // memory, so spread out they overlap the other CUs' products, and no
        // XCD runs a round of whole tiles more than the others.
        const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
        const int nfull = split > 1 ? full : total;
        const int W = min(p.plan[p.E] * p.NT, nfull), R = nfull - W;
        const int w0 = (int)((int64_t)xcd * W / 8), nw = (int)((int64_t)(xcd + 1) * W / 8) - w0;
        const int r0 = (int)((int64_t)xcd * R / 8), nr = (int)((int64_t)(xcd + 1) * R / 8) - r0;
        const int n = nw + nr;
        if (slot >= n) return;
        // remainder tiles among the XCD's slots [0, s): floor(s nr / n)
        const int c0 = (int)((int64_t)slot * nr / n), c1 = (int)((int64_t)(slot + 1) * nr / n);
        L = c1 > c0 ? W + r0 + c0 : w0 + slot - c0;
    } else {
        if (split <= 1) return;
        unit = blockIdx.x - p.main_blocks;
        if (unit >= tail * split) return;
        L = full + unit / split;
        const int c = unit % split;
        k0 = c * p.nk / split;
        k1 = (c + 1) * p.nk / split;
    }
    const TileDesc t = decode_tile(p, L, BM);
    if constexpr (BF16 && BM == 256) {
        if (t.rem) {
            gemm_tile<BF16, kRemBM, BN, EPI, WGN, KM, STG>(p, lds, t, k0, k1, unit);
            return;
        }
    }
    if constexpr (BF16 && BM == 256 && BN == 256 && WGN == 4)
        gemm_tile_pp<EPI, STG, KM>(p, lds, t, k0, k1, unit);
    else
        gemm_tile<BF16, BM, BN, EPI, WGN, KM, STG>(p, lds, t, k0, k1, unit);
#endif
}

template <bool BF16, int BM, int BN, int EPI, int WGM, int WGN>
__device__ __forceinline__ void fixup_tile(const GemmParams& p, const TileDesc& t, int w, int i0, int split) {
    typedef GemmEpilogue<BF16, BM, BN, EPI, WGM, WGN> Epi;
    constexpr int FM = Epi::FM, RA = Epi::RA, IG = Epi::IG;
    const int lane = threadIdx.x;
    typename Epi::acc_t acc[IG][FM];
    const float4* src = (const float4*)p.partial;
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < RA; ++r) acc[i][j][r] = 0.0f;
    const int tt = blockIdx.x / (Epi::NW * (Epi::FN / IG));
    for (int c = 0; c < split; ++c) {
        const int u = tt * split + c;
#pragma unroll
        for (int i = 0; i < IG; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r4 = 0; r4 < RA / 4; ++r4) {
                    const float4 v = src[Epi::partial_index(p, u, w, i0 + i, j, r4, lane)];
                    acc[i][j][4 * r4] += v.x;
                    acc[i][j][4 * r4 + 1] += v.y;
                    acc[i][j][4 * r4 + 2] += v.z;
                    acc[i][j][4 * r4 + 3] += v.w;
                }
    }
    Epi::store_cols(p, acc, i0, t.row0, t.rows, t.nt, w / WGN, w % WGN, lane);
}

// Split-K fixup: block (t, w, g) adds, in range order, the `split` partial
// accumulators of column group g of wave w of tail tile t, and applies the
// epilogue to them (with the remainder-tile layout for remainder tiles).
template <bool BF16, int BM, int BN, int EPI, int WGM, int WGN>
__global__ __launch_bounds__(64) void k_split_fixup(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef GemmEpilogue<BF16, BM, BN, EPI, WGM, WGN> Epi;
    constexpr int IG = Epi::IG, NGRP = Epi::FN / IG, NW = Epi::NW;
    const int full = p.plan[p.E + 1], split = p.plan[p.E + 2], tail = p.plan[p.E + 3];
    const int t = blockIdx.x / (NW * NGRP), w = (blockIdx.x / NGRP) % NW, i0 = (blockIdx.x % NGRP) * IG;
    if (split <= 1 || t >= tail) return;
    const TileDesc td = decode_tile(p, full + t, BM);
    if constexpr (BF16 && BM == 256 && WGM == 2) {
        if (td.rem) {
            fixup_tile<BF16, kRemBM, BN, EPI, 2, WGN>(p, td, w, i0, split);
            return;
        }
    }
    fixup_tile<BF16, BM, BN, EPI, WGM, WGN>(p, td, w, i0, split);
#endif
}

// Tile plan: prefix[e+1] = sum_{e' <= e} (whole row tiles of expert e'),
// then the split-K decision {full, split, tail} (see kSplitUnits), then at
// [E + 4, 2E + 4] the same prefix of remainder tiles.  Expert e has
// ceil(M_e / BM) whole tiles, or, with rem set and a remainder
// r = M_e mod BM in 1 .. kRemThr, floor(M_e / BM) whole tiles and
// ceil(r / kRemBM) remainder tiles.  With offsets == NULL the plan describes
// one group of uniform_rows rows and offsets_copy receives {0, uniform_rows}.
// One block of 1024 threads (E <= 1024).
// With prefix2 != NULL the same block also writes the plan of a second GEMM
// over the same groups (BM2, rem2, NT2, nk2), so two GEMMs share a launch.
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ offsets, int E, int uniform_rows,
                                                    int BM, int rem, int NT, int nk,
                                                    int32_t* __restrict__ prefix, int32_t* __restrict__ offsets_copy,
                                                    int BM2, int rem2, int NT2, int nk2,
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
    auto plan = [&](int bm, int rm, int nt, int nkk, int32_t* pre) {
        const int32_t whole = whole_tiles(M, bm, rm != 0);
        const int32_t nr = remainder_tiles(M, bm, rm != 0);
        __syncthreads();   // a previous plan's reads of scan are done
        scan[0][e] = whole;
        scan[1][e] = nr;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t v0 = e >= off ? scan[0][e - off] : 0;
            const int32_t v1 = e >= off ? scan[1][e - off] : 0;
            __syncthreads();
            scan[0][e] += v0;
            scan[1][e] += v1;
            __syncthreads();
        }
        if (e == 0) {
            pre[0] = 0;
            pre[E + 4] = 0;
        }
        if (e < E) {
            pre[e + 1] = scan[0][e];
            pre[E + 4 + e + 1] = scan[1][e];
        }
        if (e == 0) {
            const int total = (scan[0][E - 1] + scan[1][E - 1]) * nt;
            int split, tail;
            split_rule(total, nkk, split, tail);
            pre[E + 1] = total - tail;
            pre[E + 2] = split;
            pre[E + 3] = tail;
        }
    };
    plan(BM, rem, NT, nk, prefix);
    if (prefix2) plan(BM2, rem2, NT2, nk2, prefix2);
}

size_t ffn_tile_plan_ints(int E) { return 2 * (size_t)E + 5; }

// Tile counts and K slices of a grouped GEMM as launch_grouped_gemm sets them.
static bool uses_rem(bool bf16, int BM) { return MOE_GEMM_REM && bf16 && BM == 256; }

static void gemm_geometry(bool bf16, int epi, int N, int K, int BM, int BN, int& NT, int& nk, int& rem) {
    NT = epi_swiglu(epi) ? N / (BN / 2) : N / BN;
    nk = K * (bf16 ? 2 : 4) / 128;
    rem = uses_rem(bf16, BM) ? 1 : 0;
}

PlanGeom plan_geom(bool bf16, int epi, int N, int K, int BM, int BN, int32_t* pre) {
    PlanGeom g;
    gemm_geometry(bf16, epi, N, K, BM, BN, g.NT, g.nk, g.rem);
    g.BM = BM;
    g.pre = pre;
    return g;
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

GemmShape pick_gemm_shape(bool bf16, int epi, int64_t rows, int E, int N, int K) {
    const int64_t avg = E > 0 ? rows / E : rows;
    GemmShape g;
    g.BM = avg >= 384 ? 256 : (avg >= 96 ? 128 : 64);
    // long reductions (K >= 2048) take 256-row tiles from 96 rows per expert
    // on: each tile streams a long weight panel, and halving the panel reads
    // outweighs the padded rows (DeepSeek-V3 shape, 128 rows per expert on
    // average: up 2.25 -> 2.15 ms, down 1.17 -> 1.01 ms; with K = 512 / 1024
    // the down projection was 7-10 % slower, so short reductions keep 128)
    if (bf16 && K >= 2048 && avg >= 96) g.BM = 256;
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
// Waves along N of a tile: 4 for the ping-pong tiles (8 waves), else 2.
template <bool BF16, int BM, int BN, int KM = KM_NONE>
constexpr int waves_n() { return (BF16 && BM == 256 && BN == 256 && MOE_GEMM_PP) ? 4 : 2; }

// Whole tiles and split units in one launch, then the fixup when the plan
// may have a split.
template <bool BF16, int BM, int BN, int EPI, int KM = KM_NONE>
static void launch_pair(const GemmParams& p0, int grid, bool may_split, hipStream_t s) {
    constexpr int WGN = waves_n<BF16, BM, BN, KM>();
    typedef GemmEpilogue<BF16, BM, BN, EPI, 2, WGN> Epi;
    GemmParams p = p0;
    // per XCD at most ceil(whole / 8) + ceil(remainder / 8) tiles: two block
    // slots per XCD beyond the tile bound
    p.main_blocks = grid + 16;
    const dim3 g(p.main_blocks + (may_split ? kSplitUnits : 0)), b(128 * WGN);
    // the staged-output instantiation where the epilogue can stage and C
    // and ldc allow 16-byte row stores
    bool staged = false;
    if constexpr (Epi::can_stage) staged = p.ldc % 8 == 0 && ((uintptr_t)p.C & 15) == 0;
    if (staged) {
        if constexpr (Epi::can_stage) hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI, WGN, KM, true>), g, b, 0, s, p);
    } else {
        hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI, WGN, KM, false>), g, b, 0, s, p);
    }
    if (!may_split) return;
    constexpr int groups = Epi::FN / Epi::IG;
    hipLaunchKernelGGL((k_split_fixup<BF16, BM, BN, EPI, 2, WGN>), dim3(kSplitUnits / 2 * Epi::NW * groups), dim3(64),
                       0, s, p);
}

template <bool BF16, int BM, int BN>
static void launch_bmbn(int epi, const GemmParams& p, int grid, bool ms, hipStream_t s) {
    // SwiGLU tiles need an even number of MFMA blocks per wave along N (gate
    // and up blocks in pairs); gemm_shape_supported() keeps other shapes away
    constexpr bool swiglu_ok = (BN / waves_n<BF16, BM, BN>() / mfma_block<BF16>()) % 2 == 0;
    switch (epi) {
        case EPI_STORE: launch_pair<BF16, BM, BN, EPI_STORE>(p, grid, ms, s); break;
        case EPI_RELU: launch_pair<BF16, BM, BN, EPI_RELU>(p, grid, ms, s); break;
        case EPI_RELU_SAVE: launch_pair<BF16, BM, BN, EPI_RELU_SAVE>(p, grid, ms, s); break;
        case EPI_SWIGLU_SAVE:
            if constexpr (swiglu_ok) launch_pair<BF16, BM, BN, EPI_SWIGLU_SAVE>(p, grid, ms, s);
            break;
        default:
            if constexpr (swiglu_ok) launch_pair<BF16, BM, BN, EPI_SWIGLU>(p, grid, ms, s);
            break;
    }
}

// Whether launch_t has a kernel for this tile shape and epilogue.
static bool gemm_shape_supported(bool bf16, int epi, int BM, int BN) {
    if (!bf16 && BM > 128) return false;
    if (!epi_swiglu(epi)) return true;
    const int mb = bf16 ? mfma_block<true>() : mfma_block<false>();
    const int wgn = (bf16 && BM == 256 && BN == 256 && MOE_GEMM_PP) ? 4 : 2;
    return (BN / wgn / mb) % 2 == 0;
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
    int split, tail;
    split_rule((int)(total % kSplitUnits), nk, split, tail);
    return split >= 2;
}

hipError_t launch_grouped_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B0, const void* B1,
                               int64_t b_expert_stride, void* C, int64_t ldc, int N, int K, int E, int64_t max_rows,
                               const int32_t* offsets, int32_t* plan, int32_t* plan_copy, float* partial, int BM,
                               int BN, hipStream_t s, void* C2, int64_t ldc2, bool plan_ready,
                               const int32_t* arows, int64_t a_rows, int arow_div) {
    if (max_rows <= 0) return hipSuccess;
    GemmParams p;
    p.A = A; p.lda = lda; p.B0 = B0; p.B1 = B1; p.bstride = b_expert_stride;
    p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.E = offsets ? E : 1;
    int rem = 0;
    gemm_geometry(bf16, epi, N, K, BM, BN, p.NT, p.nk, rem);
    p.offsets = offsets ? offsets : plan_copy;
    p.plan = plan;
    p.partial = partial;
    p.C2 = C2;
    p.ldc2 = ldc2;
    p.rem = rem;
    p.unit_f4 = (int64_t)BM * BN / 4;
    p.ldb = 0;
    p.K1 = 0;
    p.arows = arows;
    p.a_bytes = arows ? a_rows * lda * (bf16 ? 2 : 4) : 0;
    p.arow_div = arow_div > 0 ? arow_div : 1;
    if (!gemm_shape_supported(bf16, epi, BM, BN) || (rem && !gemm_shape_supported(bf16, epi, kRemBM, BN)))
        return hipErrorInvalidValue;
    // a gathered row's 32-bit byte offset must stay below 2^31
    if (arows && (a_rows <= 0 || arow_div <= 0 || p.a_bytes >= ((int64_t)1 << 31))) return hipErrorInvalidValue;
    if (!plan_ready)
        hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, E, (int)max_rows, BM, rem, p.NT, p.nk,
                           plan, plan_copy, 0, 0, 0, 0, (int32_t*)nullptr);
    // row tiles: at most ceil(rows / BM) plus, per expert, one partial tile or
    // up to ceil(kRemThr / kRemBM) remainder tiles
    const int64_t per_expert = rem ? (kRemThr + kRemBM - 1) / kRemBM : 1;
    const int64_t m_tiles_ub = (max_rows + BM - 1) / BM + (p.E > 1 ? p.E * per_expert : per_expert);
    const int64_t grid = (m_tiles_ub * p.NT + 7) / 8 * 8;
    if (grid > 0x7fffffff - kSplitUnits - 16) return hipErrorInvalidValue;
    // With offsets == NULL the host knows the row count and launches the
    // split-K parts only when the plan has a tail; routed counts live on the
    // device.
    bool may_split = true;
    if (offsets == nullptr) {
        const int64_t whole = whole_tiles((int)max_rows, BM, rem != 0);
        const int64_t r = max_rows - whole * BM;
        const int64_t tiles = whole + (r > 0 ? (r + kRemBM - 1) / kRemBM : 0);
        may_split = plan_may_split(tiles * p.NT, p.nk);
    }
    if (bf16) launch_t<true>(epi, p, BM, BN, (int)grid, may_split, s);
    else launch_t<false>(epi, p, BM, BN, (int)grid, may_split, s);
    return hipGetLastError();
}


// ---- products with k-major operands (the backward's products through the
// weights as stored and its weight gradients)

bool grouped_gemm_nn_supported(int64_t lda, int K, int K1, int64_t ldb, int N, bool has_b1) {
    if (K <= 0 || K % 64 || K1 <= 0 || K1 > K || K1 % 64) return false;
    if ((K1 < K) != has_b1) return false;
    if (N <= 0 || N % 128 || lda % 8 || ldb % 8 || ldb < N) return false;
    if ((int64_t)K1 * ldb * 2 >= ((int64_t)1 << 31) || (int64_t)(K - K1) * ldb * 2 >= ((int64_t)1 << 31)) return false;
    if ((255 * lda + K) * 2 >= ((int64_t)1 << 31)) return false;
    return true;
}

template <int BM>
static void launch_nn_bm(const GemmParams& p, int BN, int grid, bool ms, hipStream_t s) {
    if (BN == 256) launch_pair<true, BM, 256, EPI_STORE, KM_B>(p, grid, ms, s);
    else launch_pair<true, BM, 128, EPI_STORE, KM_B>(p, grid, ms, s);
}

hipError_t launch_grouped_gemm_nn(const void* A, int64_t lda, const void* B0, const void* B1, int K1, int64_t ldb,
                                  int64_t bstride, void* C, int64_t ldc, int N, int K, int E, int64_t max_rows,
                                  const int32_t* offsets, int32_t* plan, int32_t* plan_copy, float* partial,
                                  hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (!grouped_gemm_nn_supported(lda, K, K1, ldb, N, B1 != nullptr)) return hipErrorInvalidValue;
    const GemmShape g = pick_gemm_shape(true, EPI_STORE, max_rows, offsets ? E : 1, N);
    const int BM = g.BM, BN = (N % 256 == 0) ? 256 : 128;
    GemmParams p;
    p.A = A; p.lda = lda; p.B0 = B0; p.B1 = B1; p.bstride = bstride;
    p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.E = offsets ? E : 1;
    int rem = 0;
    gemm_geometry(true, EPI_STORE, N, K, BM, BN, p.NT, p.nk, rem);
    p.offsets = offsets ? offsets : plan_copy;
    p.plan = plan;
    p.partial = partial;
    p.C2 = nullptr;
    p.ldc2 = 0;
    p.rem = rem;
    p.unit_f4 = (int64_t)BM * BN / 4;
    p.ldb = ldb;
    p.K1 = K1;
    p.arows = nullptr;
    p.a_bytes = 0;
    p.arow_div = 1;
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, E, (int)max_rows, BM, rem, p.NT, p.nk, plan,
                       plan_copy, 0, 0, 0, 0, (int32_t*)nullptr);
    const int64_t per_expert = rem ? (kRemThr + kRemBM - 1) / kRemBM : 1;
    const int64_t m_tiles_ub = (max_rows + BM - 1) / BM + (p.E > 1 ? p.E * per_expert : per_expert);
    const int64_t grid = (m_tiles_ub * p.NT + 7) / 8 * 8;
    if (grid > 0x7fffffff - kSplitUnits - 16) return hipErrorInvalidValue;
    bool may_split = true;
    if (offsets == nullptr) {
        const int64_t whole = whole_tiles((int)max_rows, BM, rem != 0);
        const int64_t r = max_rows - whole * BM;
        const int64_t tiles = whole + (r > 0 ? (r + kRemBM - 1) / kRemBM : 0);
        may_split = plan_may_split(tiles * p.NT, p.nk);
    }
    if (BM == 256) launch_nn_bm<256>(p, BN, (int)grid, may_split, s);
    else if (BM == 128) launch_nn_bm<128>(p, BN, (int)grid, may_split, s);
    else launch_nn_bm<64>(p, BN, (int)grid, may_split, s);
    return hipGetLastError();
}


}  // namespace moe
