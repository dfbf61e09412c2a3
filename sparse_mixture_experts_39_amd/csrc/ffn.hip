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
//     double buffered, one barrier per K step; the global loads for step
//     k+1 are issued before the MFMAs of step k.  16-byte chunks are XOR
//     swizzled by (r ^ (r >> 3)) & 7 so fragment reads of 8 or 16
//     consecutive rows and row writes hit distinct banks.
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

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <bool BF16, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void k_grouped_gemm(GemmParams p) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int KT = 128 / ES;              // K elements per LDS row
    constexpr int CA = BM / 32, CB = BN / 32; // 16-byte chunks per thread per tile
    static_assert(EPI != EPI_SWIGLU || (FN % 2) == 0, "SwiGLU pairs 16-row blocks");
    __shared__ __align__(16) uint8_t lds[2][(BM + BN) * 128];

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

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global source pointers of this thread's chunks
    const uint8_t* gA[CA];
    const uint8_t* gB[CB];
    int ldsA[CA], ldsB[CB];
    const int cchunk = tid & 7;
#pragma unroll
    for (int q = 0; q < CA; ++q) {
        const int r = (tid >> 3) + 32 * q;
        const int src = row0 + min(r, rows - 1);
        gA[q] = (const uint8_t*)p.A + ((int64_t)src * p.lda) * ES + cchunk * 16;
        ldsA[q] = r * 128 + ((cchunk ^ swz(r)) << 4);
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        const int r = (tid >> 3) + 32 * q;
        const uint8_t* base;
        int64_t brow;
        if constexpr (EPI == EPI_SWIGLU) {
            const int j = r >> 4;
            brow = (int64_t)nt * (BN / 2) + (j >> 1) * 16 + (r & 15);
            base = (const uint8_t*)((j & 1) ? p.B1 : p.B0);
        } else {
            brow = (int64_t)nt * BN + r;
            base = (const uint8_t*)p.B0;
        }
        gB[q] = base + ((int64_t)e * p.bstride + brow * p.K) * ES + cchunk * 16;
        ldsB[q] = (BM + r) * 128 + ((cchunk ^ swz(r)) << 4);
    }

    floatx4_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4_t ra[CA], rb[CB];
    // fragment read offsets (row part), chunk part added per sub-step
    int fa_row[FM], fb_row[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa_row[i] = wm * WM + i * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < FN; ++i) fb_row[i] = BM + wn * WN + i * 16 + (lane & 15);
    const int lg = lane >> 4;

    const int nk = p.K / KT;
#pragma unroll
    for (int q = 0; q < CA; ++q) ra[q] = *(const u32x4_t*)(gA[q]);
#pragma unroll
    for (int q = 0; q < CB; ++q) rb[q] = *(const u32x4_t*)(gB[q]);
#pragma unroll
    for (int q = 0; q < CA; ++q) *(u32x4_t*)(&lds[0][ldsA[q]]) = ra[q];
#pragma unroll
    for (int q = 0; q < CB; ++q) *(u32x4_t*)(&lds[0][ldsB[q]]) = rb[q];
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int64_t koff = (int64_t)(kt + 1) * 128;
#pragma unroll
            for (int q = 0; q < CA; ++q) ra[q] = *(const u32x4_t*)(gA[q] + koff);
#pragma unroll
            for (int q = 0; q < CB; ++q) rb[q] = *(const u32x4_t*)(gB[q] + koff);
        }
        const uint8_t* L0 = lds[cur];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 4 * s + lg;
            u32x4_t fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = fa_row[i];
                fa[i] = *(const u32x4_t*)(L0 + r * 128 + ((ch ^ swz(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int r = fb_row[i];
                fb[i] = *(const u32x4_t*)(L0 + r * 128 + ((ch ^ swz(r - BM)) << 4));
            }
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    if constexpr (BF16) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, fb[i]), __builtin_bit_cast(bf16x8_t, fa[j]), acc[i][j], 0, 0, 0);
                    } else {
                        const floatx4_t b4 = __builtin_bit_cast(floatx4_t, fb[i]);
                        const floatx4_t a4 = __builtin_bit_cast(floatx4_t, fa[j]);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[0], a4[0], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[1], a4[1], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[2], a4[2], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[3], a4[3], acc[i][j], 0, 0, 0);
                    }
                }
        }
        if (kt + 1 < nk) {
            uint8_t* Ln = lds[cur ^ 1];
#pragma unroll
            for (int q = 0; q < CA; ++q) *(u32x4_t*)(Ln + ldsA[q]) = ra[q];
#pragma unroll
            for (int q = 0; q < CB; ++q) *(u32x4_t*)(Ln + ldsB[q]) = rb[q];
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds D[n = 4*(lane/16) + r][m = lane % 16] per block
    const int m_in = lane & 15;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int pi = 0; pi < FN / 2; ++pi) {
            const int fblock = (wn * FN + 2 * pi) >> 1;
            const int f = nt * (BN / 2) + fblock * 16 + 4 * lg;
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = wm * WM + j * 16 + m_in;
                if (m >= rows) continue;
                float h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gt = acc[2 * pi][j][r], up = acc[2 * pi + 1][j][r];
                    h[r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                }
                const int64_t o = (int64_t)(row0 + m) * p.ldc + f;
                if constexpr (BF16) {
                    uint2 v;
                    v.x = f32_to_bf16_bits(h[0]) | (f32_to_bf16_bits(h[1]) << 16);
                    v.y = f32_to_bf16_bits(h[2]) | (f32_to_bf16_bits(h[3]) << 16);
                    *(uint2*)((uint16_t*)p.C + o) = v;
                } else {
                    *(float4*)((float*)p.C + o) = make_float4(h[0], h[1], h[2], h[3]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int n = nt * BN + wn * WN + i * 16 + 4 * lg;
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = wm * WM + j * 16 + m_in;
                if (m >= rows) continue;
                float v4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = acc[i][j][r];
                    if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.0f);
                    v4[r] = v;
                }
                const int64_t o = (int64_t)(row0 + m) * p.ldc + n;
                if constexpr (BF16) {
                    uint2 v;
                    v.x = f32_to_bf16_bits(v4[0]) | (f32_to_bf16_bits(v4[1]) << 16);
                    v.y = f32_to_bf16_bits(v4[2]) | (f32_to_bf16_bits(v4[3]) << 16);
                    *(uint2*)((uint16_t*)p.C + o) = v;
                } else {
                    *(float4*)((float*)p.C + o) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                }
            }
        }
    }
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
