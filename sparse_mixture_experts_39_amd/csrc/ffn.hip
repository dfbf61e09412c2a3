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
//     each wave a (BM/2) x (BN/2) tile of 16x16 MFMA blocks.
//   * MFMA operand order: the weights are source 0 and the activations
//     source 1, so the accumulator lanes hold 4 consecutive output columns of
//     one row and the epilogue stores 8 (bf16) or 16 (fp32) bytes per lane.
//   * bf16 uses v_mfma_f32_16x16x32_bf16 (one 16-byte fragment per lane = 8 k
//     values); fp32 uses four v_mfma_f32_16x16x4_f32 per 16-byte fragment.
//     The k positions inside a fragment are the same for both operands, so
//     the product is exact whatever order the unit visits them in.
//   * K is staged through LDS in 128-byte rows (64 bf16 / 32 fp32 values),
//     double buffered, one barrier per K step.  The tiles move with gfx950's
//     direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds), so no VGPRs
//     hold staged data; the loads for step k+1 are in flight during the
//     MFMAs of step k.
//     16-byte chunks are XOR swizzled by (r ^ (r >> 3)) & 7 so fragment
//     reads of 8 or 16 consecutive rows hit distinct banks.
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
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

enum { EPI_STORE = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };

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
    const int32_t* offsets; // [E+1]
    const int32_t* tile_prefix;  // [E+1]
};

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row: fragment reads
// of 8 or 16 consecutive rows at one logical chunk land in distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

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

template <bool BF16, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void k_grouped_gemm(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MB = BF16 ? 32 : 16;        // MFMA block edge (32x32x16 bf16, 16x16x4 fp32)
    constexpr int FM = WM / MB, FN = WN / MB;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int KT = 64 / ES;               // K elements per stage (64-byte rows)
    constexpr int NS = 4;                     // pipeline stages
    constexpr int STAGE = (BM + BN) * 64;     // bytes per stage
    constexpr int KS = BF16 ? 2 : 1;          // MFMA k-steps per stage
    typedef typename std::conditional<BF16, floatx16_t, floatx4_t>::type acc_t;
    static_assert(FM >= 1 && FN >= 1, "tile smaller than one MFMA block");
    static_assert(BF16 || EPI != EPI_SWIGLU || (FN % 2) == 0, "SwiGLU pairs 16-row blocks");
    __shared__ __align__(16) uint8_t lds[NS * STAGE];

    // ---- tile decode (device-side ragged plan, XCD-contiguous ranges)
    const int NT = p.NT;
    const int total = p.tile_prefix[p.E] * NT;
    const int per_xcd = (total + 7) / 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per_xcd) return;
    const int L = (blockIdx.x % 8) * per_xcd + slot;
    if (L >= total) return;
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.tile_prefix[mid] * NT <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int tiles_e = p.tile_prefix[e + 1] - p.tile_prefix[e];
    const int local = L - p.tile_prefix[e] * NT;
    constexpr int NG = 8;
    const int grp = local / (tiles_e * NG);
    const int inside = local - grp * tiles_e * NG;
    const int mt = inside % tiles_e;
    const int nt = grp * NG + inside / tiles_e;
    const int row0 = p.offsets[e] + mt * BM;
    const int rows = min(BM, p.offsets[e + 1] - row0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int wm = wave >> 1, wn = wave & 1;

    // ---- direct-to-LDS loads.  A stage holds the A rows then the B rows of
    // one K slice, 64 bytes per row, filled in 1 KB groups of 16 rows; one
    // buffer_load_dwordx4 ... lds of a wave fills one group, lane l landing
    // at byte 16*l, i.e. row 16*g + l/4, physical chunk l%4.  The lane
    // fetches logical chunk (l%4) ^ swz(row): the swizzle is applied on the
    // global side.  Addresses are buffer descriptors (SGPRs) holding the
    // tile's base and extent, a 32-bit lane offset, and the K offset in an
    // SGPR; a read past the extent returns zeros instead of touching memory.
    constexpr int GA = BM / 16, GB = BN / 16, GPW = (GA + GB) / 4;  // groups per wave
    static_assert((GA + GB) % 4 == 0, "groups split evenly over 4 waves");
    constexpr int kRsrcWord3 = 0x00020000;
    const int64_t brow_base = EPI == EPI_SWIGLU ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;
    const int b_rows = EPI == EPI_SWIGLU ? BN / 2 : BN;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.A + (int64_t)row0 * p.lda * ES), (short)0,
        (int)(((int64_t)(rows - 1) * p.lda + p.K) * ES), kRsrcWord3);
    const int64_t boff = ((int64_t)e * p.bstride + brow_base * p.K) * ES;
    const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.B0 + boff), (short)0, (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)(EPI == EPI_SWIGLU ? p.B1 : p.B0) + boff), (short)0,
        (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
    uint32_t voff[GPW];
    int src_of[GPW];  // 0: A, 1: B0, 2: B1 (wave-uniform)
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const int g = wave * GPW + q;
        if (g < GA) {
            const int r = 16 * g + (lane >> 2);
            const int lc = (lane & 3) ^ swz(r);
            src_of[q] = 0;
            voff[q] = (uint32_t)(min(r, rows - 1) * (int)p.lda * ES + lc * 16);
        } else {
            const int j = g - GA;                          // 16-row block of B
            const int r = 16 * j + (lane >> 2);
            const int lc = (lane & 3) ^ swz(r);
            int rr;
            if constexpr (EPI == EPI_SWIGLU) {
                src_of[q] = (j & 1) ? 2 : 1;               // gate / up blocks alternate
                rr = (j >> 1) * 16 + (lane >> 2);
            } else {
                src_of[q] = 1;
                rr = r;
            }
            voff[q] = (uint32_t)(rr * p.K * ES + lc * 16);
        }
    }
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    auto issue = [&](int kt, int stage) {
        const int koff = kt * 64;
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const int g = wave * GPW + q;
            lds_ptr_t dst = (lds_ptr_t)(&lds[stage * STAGE + g * 1024]);
            if (src_of[q] == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, dst, 16, voff[q], koff, 0, 0);
            else if (src_of[q] == 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB0, dst, 16, voff[q], koff, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB1, dst, 16, voff[q], koff, 0, 0);
        }
    };

    acc_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < (BF16 ? 16 : 4); ++r) acc[i][j][r] = 0.0f;

    // Fragment reads.  bf16 (32x32x16): lane l takes row l % 32 of a 32-row
    // block at chunk 2*s + l/32 for k-step s (8 k values per lane).  fp32
    // (16x16x4): lane l takes row l % 16 at chunk l/16 (4 k values, four
    // MFMAs).  Weights are MFMA source 0 (rows = output columns n),
    // activations source 1 (columns = token rows m).
    constexpr int NF = KS * (FM + FN);       // fragments per stage
    int f_off[NF];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
        const int ch = BF16 ? (2 * s2 + (lane >> 5)) : (lane >> 4);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = wm * WM + i * MB + (lane & (MB - 1));
            f_off[s2 * (FM + FN) + i] = r * 64 + ((ch ^ swz(r)) << 4);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int r = wn * WN + i * MB + (lane & (MB - 1));
            f_off[s2 * (FM + FN) + FM + i] = (BM + r) * 64 + ((ch ^ swz(r)) << 4);
        }
    }
    auto read_frags = [&](int stage, u32x4_t* f) {
        const uint8_t* Lb = &lds[stage * STAGE];
#pragma unroll
        for (int i = 0; i < NF; ++i) f[i] = *(const u32x4_t*)(Lb + f_off[i]);
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
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
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

    // Pipeline over K stages kt = 0 .. nk-1, stage kt in buffer kt % NS.
    // Loads run NS stages ahead of the MFMAs.  Iteration kt holds stage kt's
    // fragments in registers and
    //   1. waits until this wave's loads of stage kt+1 have landed,
    //   2. barrier: every wave's stage kt+1 is visible, and every wave has
    //      its stage-kt fragments in registers, so buffer kt % NS is free,
    //   3. refills buffer kt % NS with stage kt+NS,
    //   4. reads stage kt+1's fragments  while  5. MFMAs consume stage kt's.
    const int nk = p.K / KT;
    u32x4_t f0[NF], f1[NF];
    auto wait_pending = [&](int pending) {      // leave `pending` stages in flight
        if (pending >= 3) wait_vmcnt<3 * GPW>();
        else if (pending == 2) wait_vmcnt<2 * GPW>();
        else if (pending == 1) wait_vmcnt<GPW>();
        else wait_vmcnt<0>();
    };
    const int pre = nk < NS ? nk : NS;
    for (int s = 0; s < pre; ++s) issue(s, s);
    wait_pending(pre - 1);
    lds_barrier();
    read_frags(0, f0);
    int kt = 0;
    auto step = [&](u32x4_t* f, u32x4_t* f_n) {
        const int issued_last = min(kt + NS - 1, nk - 1);   // loads issued: stages 0 .. issued_last
        if (kt + 1 < nk) wait_pending(issued_last - (kt + 1));
        lds_barrier();
        if (kt + NS < nk) issue(kt + NS, kt % NS);
        if (kt + 1 < nk) read_frags((kt + 1) % NS, f_n);
        __builtin_amdgcn_sched_barrier(0);
        mma(f);
        __builtin_amdgcn_sched_barrier(0);
        ++kt;
    };
    while (kt + 1 < nk) {
        step(f0, f1);
        step(f1, f0);
    }
    if (kt < nk) step(f0, f1);

    // ---- epilogue.  bf16 blocks (32x32): lane l, element r = 4q + t holds
    // D[n = 8q + 4(l/32) + t][m = l % 32].  fp32 blocks (16x16): element t
    // holds D[n = 4(l/16) + t][m = l % 16].  Either way a lane owns 4
    // consecutive output columns of one row per (q) and stores them at once.
    auto store4 = [&](int m, int64_t col, const float* v) {
        const int64_t o = (int64_t)(row0 + m) * p.ldc + col;
        if constexpr (BF16) {
            uint2 w;
            w.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
            w.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
            *(uint2*)((uint16_t*)p.C + o) = w;
        } else {
            *(float4*)((float*)p.C + o) = make_float4(v[0], v[1], v[2], v[3]);
        }
    };
    auto silu_mul = [](float gt, float up) { return gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up; };
    if constexpr (BF16) {
        const int h = lane >> 5;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = wm * WM + j * 32 + (lane & 31);
            if (m >= rows) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int blk = wn * (WN / 32) + i;              // 32-row block of the B tile
                if constexpr (EPI == EPI_SWIGLU) {
                    // rows 0-15 of the block are gate units, rows 16-31 the
                    // up units of the same 16 hidden units: q and q+2 pair up
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = silu_mul(acc[i][j][4 * q + t], acc[i][j][4 * (q + 2) + t]);
                        store4(m, (int64_t)nt * (BN / 2) + blk * 16 + 8 * q + 4 * h, v);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            float x = acc[i][j][4 * q + t];
                            if constexpr (EPI == EPI_RELU) x = fmaxf(x, 0.0f);
                            v[t] = x;
                        }
                        store4(m, (int64_t)nt * BN + blk * 32 + 8 * q + 4 * h, v);
                    }
                }
            }
        }
    } else {
        const int lg = lane >> 4;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = wm * WM + j * 16 + (lane & 15);
            if (m >= rows) continue;
            if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int pi = 0; pi < FN / 2; ++pi) {
                    const int fblock = (wn * FN + 2 * pi) >> 1;    // 16-row blocks alternate gate / up
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = silu_mul(acc[2 * pi][j][t], acc[2 * pi + 1][j][t]);
                    store4(m, (int64_t)nt * (BN / 2) + fblock * 16 + 4 * lg, v);
                }
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float x = acc[i][j][t];
                        if constexpr (EPI == EPI_RELU) x = fmaxf(x, 0.0f);
                        v[t] = x;
                    }
                    store4(m, (int64_t)nt * BN + wn * WN + i * 16 + 4 * lg, v);
                }
            }
        }
    }
#endif
}

// Tile plan: prefix[e+1] = sum_{e' <= e} ceil(M_e' / BM).  With offsets == NULL
// the plan describes one group of uniform_rows rows and offsets_copy receives
// {0, uniform_rows}.  One block of 1024 threads (E <= 1024).
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ offsets, int E, int uniform_rows,
                                                    int BM, int32_t* __restrict__ prefix,
                                                    int32_t* __restrict__ offsets_copy) {
    __shared__ int32_t scan[1024];
    const int e = threadIdx.x;
    int32_t n = 0;
    if (offsets == nullptr) {
        if (e == 0) {
            offsets_copy[0] = 0;
            offsets_copy[1] = uniform_rows;
            n = (uniform_rows + BM - 1) / BM;
        }
        E = 1;
    } else if (e < E) {
        const int32_t M = offsets[e + 1] - offsets[e];
        n = (M + BM - 1) / BM;
    }
    scan[e] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = e >= off ? scan[e - off] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    if (e == 0) prefix[0] = 0;
    if (e < E) prefix[e + 1] = scan[e];
}

size_t ffn_tile_plan_ints(int E) { return (size_t)(E + 1) + 2; }

void launch_tile_plan(const int32_t* offsets, int E, int uniform_rows, int BM, int32_t* tile_prefix,
                      int32_t* offsets_copy, hipStream_t s) {
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, E, uniform_rows, BM, tile_prefix,
                       offsets_copy);
}

GemmShape pick_gemm_shape(bool bf16, int epi, int64_t rows, int E, int N) {
    (void)bf16;
    const int64_t avg = E > 0 ? rows / E : rows;
    GemmShape g;
    g.BM = avg >= 384 ? 256 : (avg >= 96 ? 128 : 64);
    // output columns per tile for BN = 256 / 128 / 64 (SwiGLU tiles hold gate
    // and up rows, so they produce half as many columns)
    const int div = epi == EPI_SWIGLU ? 2 : 1;
    g.BN = (N % (256 / div) == 0) ? 256 : (N % (128 / div) == 0 ? 128 : 64);
    return g;
}

template <bool BF16, int BM, int BN>
static hipError_t launch_bmbn(int epi, const GemmParams& p, int grid, hipStream_t s) {
    switch (epi) {
        case EPI_STORE:
            hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI_STORE>), dim3(grid), dim3(256), 0, s, p);
            break;
        case EPI_RELU:
            hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI_RELU>), dim3(grid), dim3(256), 0, s, p);
            break;
        default:
            hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI_SWIGLU>), dim3(grid), dim3(256), 0, s, p);
            break;
    }
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_t(int epi, const GemmParams& p, int BM, int BN, int grid, hipStream_t s) {
    if (BN == 256) {
        if (BM == 256) return launch_bmbn<BF16, 256, 256>(epi, p, grid, s);
        if (BM == 128) return launch_bmbn<BF16, 128, 256>(epi, p, grid, s);
        return launch_bmbn<BF16, 64, 256>(epi, p, grid, s);
    }
    if (BN == 128) {
        if (BM == 256) return launch_bmbn<BF16, 256, 128>(epi, p, grid, s);
        if (BM == 128) return launch_bmbn<BF16, 128, 128>(epi, p, grid, s);
        return launch_bmbn<BF16, 64, 128>(epi, p, grid, s);
    }
    if (BM == 256) return launch_bmbn<BF16, 256, 64>(epi, p, grid, s);
    if (BM == 128) return launch_bmbn<BF16, 128, 64>(epi, p, grid, s);
    return launch_bmbn<BF16, 64, 64>(epi, p, grid, s);
}

hipError_t launch_grouped_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B0, const void* B1,
                               int64_t b_expert_stride, void* C, int64_t ldc, int N, int K, int E, int64_t max_rows,
                               const int32_t* offsets, const int32_t* tile_prefix, int BM, int BN, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    GemmParams p;
    p.A = A; p.lda = lda; p.B0 = B0; p.B1 = B1; p.bstride = b_expert_stride;
    p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.E = E;
    p.NT = epi == EPI_SWIGLU ? N / (BN / 2) : N / BN;
    p.offsets = offsets; p.tile_prefix = tile_prefix;
    const int64_t m_tiles_ub = (max_rows + BM - 1) / BM + (E > 1 ? E : 0);
    int64_t grid = m_tiles_ub * p.NT;
    grid = (grid + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    return bf16 ? launch_t<true>(epi, p, BM, BN, (int)grid, s) : launch_t<false>(epi, p, BM, BN, (int)grid, s);
}

}  // namespace moe
