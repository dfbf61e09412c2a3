// Backward pass of the MoE FFN layer on gfx950: the kernels that are not the
// two input-gradient products (those run on the forward's grouped GEMM in
// ffn.hip, against transposed weight copies made here).
//
// The layer trains by ordinary backpropagation through the experts each
// token went to, with the top-k choice held constant; masked experts get
// exactly zero gradient and the selected logits a nonzero one (Shazeer et al.
// reading notes, section 2.1 key points; CS25 "Lecture29" notes, Q&A
// "Gradient flow and training cost").
//
//   k_transpose      weight copies with the other dimension contiguous
//   k_bwd_rows       per kept row r of assignment a = (t, j): dy_perm[r] =
//                    g_a dY[t] and the gate gradient dg_a = <dY[t], y_perm[r]>
//   k_bwd_act        SwiGLU / ReLU derivative: (dh, a, u) -> da | du and h
//   k_gemm_tn        ragged-K grouped GEMM C_e = A_e^T B_e over the rows of
//                    each expert: the expert weight gradients (MFMA; bf16
//                    256 x 256 tiles in k_gemm_wgrad, persistent)
//   k_bwd_router     logit gradient dz of every token from dg and the gates
//   k_bwd_dx         token gradient: residual + routed rows in slot order +
//                    shared expert + dz W_r
//   k_bwd_wr_few /
//   k_bwd_wr_mma /
//   k_bwd_wr_sum     router gradients dW_r = dz^T x and db = sum_t dz, in a
//                    fixed order over token chunks
//
// Every reduction has one fixed order, so results are bitwise reproducible.
// This file is compiled with -ffp-contract=off so the router recomputation
// matches the forward's logits bit for bit.
#include <hip/hip_runtime.h>

#include "canon_math.h"
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

template <bool BF16>
__device__ __forceinline__ void store_act(void* p, int64_t i, float v) {
    if constexpr (BF16) ((uint16_t*)p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    else ((float*)p)[i] = v;
}

// 8 consecutive activations from element i (i and the row stride multiples
// of 8: one 16-byte access for bf16, two for fp32), exact in fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, int64_t i, float* v) {
    if constexpr (BF16) {
        const u32x4_t w = *(const u32x4_t*)((const uint16_t*)p + i);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[2 * h] = __uint_as_float(w[h] << 16);
            v[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
        }
    } else {
        const float4 a = *(const float4*)((const float*)p + i), b = *(const float4*)((const float*)p + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}
template <bool BF16>
__device__ __forceinline__ void store8(void* p, int64_t i, const float* v) {
    if constexpr (BF16) {
        u32x4_t w;
#pragma unroll
        for (int h = 0; h < 4; ++h) w[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
        *(u32x4_t*)((uint16_t*)p + i) = w;
    } else {
        *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)((float*)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// Fixed-order sum over the 256 threads of a block (wave shuffles, then the
// four wave totals in order).  Every thread gets the total.
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier after this wave's LDS operations have completed; global
// loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

// dst[b][c][coff + r] = src[b][r][c] for r < R, c < C (both multiples of
// 64).  4-byte elements: one element per access through a 64 x 65 LDS tile.
__global__ __launch_bounds__(256) void k_transpose(const float* __restrict__ src, int R, int C, int64_t sbatch,
                                                   float* __restrict__ dst, int64_t ldd, int64_t dbatch, int coff) {
    __shared__ float tile[64][65];
    const int b = blockIdx.z;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const float* s = src + (int64_t)b * sbatch;
    float* d = dst + (int64_t)b * dbatch;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) tile[i][tx] = s[(int64_t)(r0 + i) * C + c0 + tx];
    __syncthreads();
    for (int i = ty; i < 64; i += 4) d[(int64_t)(c0 + i) * ldd + coff + r0 + tx] = tile[tx][i];
}

// 2-byte elements, 16 bytes per access: a 64 x 64 tile goes through LDS
// with its 16-byte column groups at slot g ^ ((r >> 3) & 7) in row r, so
// the row-wise stores and the column-wise gathers both spread over banks.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ src, int R, int C, int64_t sbatch,
                                                     uint16_t* __restrict__ dst, int64_t ldd, int64_t dbatch,
                                                     int coff) {
    __shared__ __align__(16) uint16_t tile[64 * 64];
    const int b = blockIdx.z;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const uint16_t* s = src + (int64_t)b * sbatch;
    uint16_t* d = dst + (int64_t)b * dbatch;
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (t >> 3) + 32 * h, g = t & 7;
        const u32x4_t v = *(const u32x4_t*)(s + (int64_t)(r0 + r) * C + c0 + g * 8);
        *(u32x4_t*)(tile + r * 64 + ((g ^ ((r >> 3) & 7)) << 3)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int oc = (t >> 3) + 32 * h, rg = t & 7;     // output row oc, source rows rg*8 .. +7
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ra = rg * 8 + 2 * q, rb = ra + 1;
            const uint32_t lo = tile[ra * 64 + ((((oc >> 3) ^ ((ra >> 3) & 7)) << 3) | (oc & 7))];
            const uint32_t hi = tile[rb * 64 + ((((oc >> 3) ^ ((rb >> 3) & 7)) << 3) | (oc & 7))];
            v[q] = lo | (hi << 16);
        }
        *(u32x4_t*)(d + (int64_t)(c0 + oc) * ldd + coff + r0 + rg * 8) = v;
    }
}

void launch_transpose(const void* src, int B, int R, int C, int64_t sbatch, void* dst, int64_t ldd, int64_t dbatch,
                      int coff, int elem_bytes, hipStream_t s) {
    if (B <= 0 || R <= 0 || C <= 0) return;
    // consecutive blocks take consecutive source row blocks, so the blocks
    // in flight write one stretch of each destination row (a power-of-two
    // destination stride would otherwise land them all on one channel)
    dim3 grid(R / 64, C / 64, B);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, s, (const uint16_t*)src, R, C, sbatch, (uint16_t*)dst,
                           ldd, dbatch, coff);
    else
        hipLaunchKernelGGL(k_transpose, grid, dim3(256), 0, s, (const float*)src, R, C, sbatch, (float*)dst, ldd,
                           dbatch, coff);
}

// One block per permuted row r < offsets[E]; a = perm_src[r], t = a / slots.
template <bool BF16>
__global__ __launch_bounds__(256) void k_bwd_rows(const void* __restrict__ dy, const void* __restrict__ y_perm,
                                                  const int32_t* __restrict__ perm_src,
                                                  const int32_t* __restrict__ offsets, int E,
                                                  const float* __restrict__ gates, int slots, int d,
                                                  void* __restrict__ dy_perm, float* __restrict__ dg) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    if (r >= offsets[E]) return;
    const int a = perm_src[r];
    const int t = a / slots;
    const float g = gates[a];
    float acc = 0.0f;
    if (d % 8 == 0 && ((((uintptr_t)dy) | ((uintptr_t)y_perm) | ((uintptr_t)dy_perm)) & 15) == 0) {
        // 8 consecutive columns per thread and step (16-byte accesses)
        for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
            float v[8], y[8], o[8];
            load8<BF16>(dy, (int64_t)t * d + c, v);
            load8<BF16>(y_perm, (int64_t)r * d + c, y);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc += v[u] * y[u];
                o[u] = g * v[u];
            }
            store8<BF16>(dy_perm, (int64_t)r * d + c, o);
        }
    } else {
        for (int c = threadIdx.x; c < d; c += 256) {
            const float v = load_act<BF16>(dy, (int64_t)t * d + c);
            acc += v * load_act<BF16>(y_perm, (int64_t)r * d + c);
            store_act<BF16>(dy_perm, (int64_t)r * d + c, g * v);
        }
    }
    const float tot = block_sum256(acc, red);
    if (threadIdx.x == 0) dg[a] = tot;
}

__global__ void k_zero_f32(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

void launch_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
}

void launch_bwd_rows(bool bf16, const void* dy, const void* y_perm, const int32_t* perm_src, const int32_t* offsets,
                     int E, const float* gates, int slots, int d, int64_t max_rows, void* dy_perm, float* dg,
                     hipStream_t s) {
    if (max_rows <= 0) return;
    if (bf16)
        hipLaunchKernelGGL(k_bwd_rows<true>, dim3((unsigned)max_rows), dim3(256), 0, s, dy, y_perm, perm_src, offsets,
                           E, gates, slots, d, dy_perm, dg);
    else
        hipLaunchKernelGGL(k_bwd_rows<false>, dim3((unsigned)max_rows), dim3(256), 0, s, dy, y_perm, perm_src,
                           offsets, E, gates, slots, d, dy_perm, dg);
}

// Activation derivative on rows < rows_end (= offsets[E], or n_rows when
// offsets is NULL), 4 columns per thread; a and u have row stride ld_au.
// SwiGLU: h = SiLU(a) u,
// da = dh u s (1 + a (1 - s)) with s = sigmoid(a), du = dh SiLU(a); ReLU:
// h = relu(a), da = dh [a > 0].  da goes to dadu[r][0..F), du to
// dadu[r][F..2F).
template <bool BF16, bool SWIGLU>
__global__ __launch_bounds__(256) void k_bwd_act(const void* __restrict__ dh, const void* __restrict__ a_in,
                                                 const void* __restrict__ u_in, int64_t ld_au,
                                                 const int32_t* __restrict__ offsets, int E, int n_rows, int F,
                                                 void* __restrict__ dadu, void* __restrict__ h_out) {
    const int64_t rows_end = offsets ? offsets[E] : n_rows;
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int64_t r = i4 / F;
    if (r >= rows_end) return;
    const int c = (int)(i4 - r * F);
    const int ldo = SWIGLU ? 2 * F : F;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t i = i4 + q;
        const int64_t ia = r * ld_au + c + q;
        const float g = load_act<BF16>(dh, i);
        const float av = load_act<BF16>(a_in, ia);
        if constexpr (SWIGLU) {
            const float uv = load_act<BF16>(u_in, ia);
            const float sg = 1.0f / (1.0f + __expf(-av));
            const float silu = av * sg;
            store_act<BF16>(dadu, r * ldo + c + q, g * uv * sg * (1.0f + av * (1.0f - sg)));
            store_act<BF16>(dadu, r * ldo + F + c + q, g * silu);
            store_act<BF16>(h_out, i, silu * uv);
        } else {
            store_act<BF16>(dadu, r * ldo + c + q, av > 0.0f ? g : 0.0f);
            store_act<BF16>(h_out, i, av > 0.0f ? av : 0.0f);
        }
    }
}

void launch_bwd_act(bool bf16, bool swiglu, const void* dh, const void* a, const void* u, int64_t ld_au,
                    const int32_t* offsets, int E, int64_t max_rows, int F, void* dadu, void* h, hipStream_t s) {
    const int64_t n4 = max_rows * F / 4;
    if (n4 <= 0) return;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    const int nr = (int)max_rows;
#define MOE_ACT_ARGS dh, a, u, ld_au, offsets, E, nr, F, dadu, h
    if (bf16) {
        if (swiglu) hipLaunchKernelGGL((k_bwd_act<true, true>), grid, dim3(256), 0, s, MOE_ACT_ARGS);
        else hipLaunchKernelGGL((k_bwd_act<true, false>), grid, dim3(256), 0, s, MOE_ACT_ARGS);
    } else {
        if (swiglu) hipLaunchKernelGGL((k_bwd_act<false, true>), grid, dim3(256), 0, s, MOE_ACT_ARGS);
        else hipLaunchKernelGGL((k_bwd_act<false, false>), grid, dim3(256), 0, s, MOE_ACT_ARGS);
    }
#undef MOE_ACT_ARGS
}

// ---------------------------------------------------------------------------
// Ragged-K grouped GEMM for the weight gradients:
//   C_e[m][n] = sum over rows r in [off[e], off[e+1]) of A[r][m] B[r][n]
// A [rows][lda], B [rows][ldb] (m, n contiguous), C_e [M][N] at C + e M N,
// fp32 accumulation, one rounding to the act dtype at the end.  An expert
// with no rows gets zeros.  128 x 128 tiles, 256 threads as 2 x 2 waves of
// 64 x 64, K (= rows) in chunks staged through two LDS buffers from
// registers, so the next chunk's loads are in flight during the MFMAs.
//
// bf16: the 16x16x32 MFMA wants 8 consecutive k of one row m per lane, so a
// chunk of 64 rows is written to LDS transposed, as [m][64 k] with 16-byte
// k-groups at physical slot g ^ (m & 7) ^ ((m >> 3) & 7): the fragment reads
// (16 consecutive m, one group) and the transposed writes (m = 8 i + j over
// lanes i) both spread over all banks.  A thread loads an 8 x 8 block (8
// rows, 8 columns) and transposes it in registers.
// fp32: the 16x16x4 MFMA takes one k per lane, so chunks of 32 rows stay
// [k][m] in LDS (rows padded to 144 floats).
// ---------------------------------------------------------------------------
struct TnParams {
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    void* C;
    int M, N, E;
    int tiles_m, tiles_n;
    const int32_t* offsets;
};

template <bool BF16>
__global__ __launch_bounds__(256) void k_gemm_tn(TnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BM = 128, BN = 128;
    constexpr int KC = BF16 ? 64 : 32;                     // rows per chunk
    constexpr int OPB = BF16 ? BM * KC * 2 : KC * 144 * 4; // bytes per operand per buffer
    __shared__ __align__(16) uint8_t lds[2 * 2 * OPB];
    const int tile = blockIdx.x;
    const int per_e = p.tiles_m * p.tiles_n;
    const int e = tile / per_e;
    const int tm = (tile - e * per_e) / p.tiles_n, tn = tile - e * per_e - tm * p.tiles_n;
    const int m_base = tm * BM, n_base = tn * BN;
    const int lo = p.offsets[e], hi = p.offsets[e + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int nchunks = (hi - lo + KC - 1) / KC;

    if constexpr (BF16) {
        // load unit: operand (tid < 128: A, else B), 8 columns from col0, 8 rows from k0
        const bool isA = tid < 128;
        const int u = tid & 127;
        const int cg = u & 15, kq = u >> 4;
        const int col0 = cg * 8;
        const int gcol = (isA ? m_base : n_base) + col0;
        const bool col_ok = gcol < (isA ? p.M : p.N);
        const uint16_t* base = (const uint16_t*)(isA ? p.A : p.B);
        const int64_t ld = isA ? p.lda : p.ldb;
        u32x4_t st[8];
        auto load = [&](int ch) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = lo + ch * KC + kq * 8 + i;
                if (col_ok && r < hi) st[i] = *(const u32x4_t*)(base + (int64_t)r * ld + gcol);
                else st[i] = u32x4_t{0u, 0u, 0u, 0u};
            }
        };
        auto put = [&](int buf) {
            uint8_t* dst = lds + (size_t)(buf * 2 + (isA ? 0 : 1)) * OPB;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int m = col0 + j;
                u32x4_t v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t x0 = st[2 * q][j >> 1], x1 = st[2 * q + 1][j >> 1];
                    v[q] = (j & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
                }
                const int slot = kq ^ (m & 7) ^ ((m >> 3) & 7);
                *(u32x4_t*)(dst + m * 128 + slot * 16) = v;
            }
        };
        if (nchunks > 0) {
            load(0);
            put(0);
        }
        __syncthreads();
        for (int ch = 0; ch < nchunks; ++ch) {
            const int buf = ch & 1;
            if (ch + 1 < nchunks) load(ch + 1);
            const uint8_t* sa = lds + (size_t)(buf * 2) * OPB;
            const uint8_t* sb = lds + (size_t)(buf * 2 + 1) * OPB;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int g = ks * 4 + (lane >> 4);
                u32x4_t fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * 64 + i * 16 + (lane & 15);
                    fa[i] = *(const u32x4_t*)(sa + m * 128 + ((g ^ (m & 7) ^ ((m >> 3) & 7)) * 16));
                    const int n = wn * 64 + i * 16 + (lane & 15);
                    fb[i] = *(const u32x4_t*)(sb + n * 128 + ((g ^ (n & 7) ^ ((n >> 3) & 7)) * 16));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[i]),
                                                                            __builtin_bit_cast(bf16x8_t, fa[j]),
                                                                            acc[i][j], 0, 0, 0);
            }
            if (ch + 1 < nchunks) put(buf ^ 1);
            __syncthreads();
        }
    } else {
        // fp32: 32 rows x 128 columns per operand and chunk, 4 float4 loads
        // per thread per operand (row tid/32 + 8 i, columns 4 (tid % 32))
        const int c4 = (tid & 31) * 4, r0 = tid >> 5;
        floatx4_t sta[4], stb[4];
        const bool a_ok = m_base + c4 < p.M, b_ok = n_base + c4 < p.N;
        auto load = [&](int ch) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = lo + ch * KC + r0 + 8 * i;
                const bool rok = r < hi;
                sta[i] = (rok && a_ok) ? *(const floatx4_t*)((const float*)p.A + (int64_t)r * p.lda + m_base + c4)
                                       : floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                stb[i] = (rok && b_ok) ? *(const floatx4_t*)((const float*)p.B + (int64_t)r * p.ldb + n_base + c4)
                                       : floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        };
        auto put = [&](int buf) {
            float* da = (float*)(lds + (size_t)(buf * 2) * OPB);
            float* db = (float*)(lds + (size_t)(buf * 2 + 1) * OPB);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *(floatx4_t*)(da + (r0 + 8 * i) * 144 + c4) = sta[i];
                *(floatx4_t*)(db + (r0 + 8 * i) * 144 + c4) = stb[i];
            }
        };
        if (nchunks > 0) {
            load(0);
            put(0);
        }
        __syncthreads();
        for (int ch = 0; ch < nchunks; ++ch) {
            const int buf = ch & 1;
            if (ch + 1 < nchunks) load(ch + 1);
            const float* sa = (const float*)(lds + (size_t)(buf * 2) * OPB);
            const float* sb = (const float*)(lds + (size_t)(buf * 2 + 1) * OPB);
#pragma unroll
            for (int ks = 0; ks < KC / 4; ++ks) {
                const int k = ks * 4 + (lane >> 4);
                float fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[i] = sa[k * 144 + wm * 64 + i * 16 + (lane & 15)];
                    fb[i] = sb[k * 144 + wn * 64 + i * 16 + (lane & 15)];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[i], fa[j], acc[i][j], 0, 0, 0);
            }
            if (ch + 1 < nchunks) put(buf ^ 1);
            __syncthreads();
        }
    }
    // lane holds C[m = .. + (lane & 15)][n = .. + 4 (lane >> 4) + t] of block (i = n block, j = m block)
    void* Ce = (uint8_t*)p.C + (size_t)e * p.M * p.N * (BF16 ? 2 : 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m_base + wm * 64 + j * 16 + (lane & 15);
        if (m >= p.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n_base + wn * 64 + i * 16 + 4 * (lane >> 4);
            if (n >= p.N) continue;
            const int64_t o = (int64_t)m * p.N + n;
            if constexpr (BF16) {
                uint2 w;
                w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(uint2*)((uint16_t*)Ce + o) = w;
            } else {
                *(floatx4_t*)((float*)Ce + o) = acc[i][j];
            }
        }
    }
#endif
}

// Parameters of the two 256 x 256 bf16 products below.
//   TN (weight gradients, k_gemm_wgrad): C_e[M][N] = sum over the expert's rows r of
//       A[r][m] B[r][n] (A, B row-major, m / n contiguous), C_e at e M N.
//   NN (input gradients without weight transposes, k_gemm_nn256): C[r][n] = sum_k
//       A[r][k] B_e[k][n] for the rows r of expert e (ragged), A row-major
//       with k contiguous, B_e = B0 + e bstride for k < K1 and
//       B1 + e bstride (row k - K1) beyond, both [rows][N] with n contiguous;
//       prefix[E+1] holds the experts' 256-row tile counts, summed.
struct XnParams {
    const void* A;
    int64_t lda;
    const void* B0;
    const void* B1;
    int64_t ldb;
    int64_t bstride;
    void* C;
    int64_t ldc;
    int M, N, K, K1, E;
    int tiles_m, tiles_n;
    const int32_t* offsets;
    const int32_t* prefix;
};

// NN product, bf16, 256 x 256 tiles, 512 threads: 8 waves of 64 (m) x 128
// (n), so a wave holds 128 accumulator registers and two waves share each
// SIMD; chunks of 64 k through two LDS buffers of 64 KB.  Threads 0-255
// stage 8 rows x one k-group of A per chunk as they are, threads 256-511 an
// 8 x 8 block of B, written transposed into LDS (the schedule is given at
// the main loop).  Weight rows past K1 come from B1.  Blocks map to tiles
// XCD by XCD, so the tiles of one XCD share an expert's weights in L2.
__global__ __launch_bounds__(512) void k_gemm_nn256(XnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BM = 256, KC = 64;
    constexpr int OPB = BM * KC * 2;
    // staged output: 8 waves x 64 rows of 256 bytes, rows padded by 16 bytes
    constexpr int SPITCH = 128 * 2 + 16, SBYTES = 8 * 64 * SPITCH;
    __shared__ __align__(16) uint8_t lds[2 * 2 * OPB > SBYTES ? 2 * 2 * OPB : SBYTES];
    // tiles: (sum of the experts' row tiles) x tiles_n.  Groups of GM row tiles: the 32 CUs of an XCD run 4 row
    // tiles x 8 column tiles at a time, so each staged chunk of A is fetched
    // once per 8 tiles and each chunk of B once per 4.
    constexpr int GM = 4;
    const int mt_all = p.prefix[p.E];
    const int ntiles = mt_all * p.tiles_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (tile >= ntiles) return;
    int e, tm, tn;
    {
        const int grp = tile / (GM * p.tiles_n);
        const int gm = min(mt_all - grp * GM, GM);
        const int in = tile - grp * GM * p.tiles_n;
        const int mt = grp * GM + in % gm;
        tn = in / gm;
        int lo_e = 0, hi_e = p.E;                 // expert: prefix[e] <= mt < prefix[e+1]
        while (hi_e - lo_e > 1) {
            const int mid = (lo_e + hi_e) >> 1;
            if (p.prefix[mid] <= mt) lo_e = mid; else hi_e = mid;
        }
        e = lo_e;
        tm = mt - p.prefix[e];
    }
    e = __builtin_amdgcn_readfirstlane(e);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int lo = p.offsets[e], hi = p.offsets[e + 1];
    // first row of the tile
    const int m_base = lo + tm * BM, n_base = tn * BM;
    const int rows_tile = min(BM, hi - m_base);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nch = p.K / KC;

    // staging: operand op (0: A, 1: B) of this thread.  Transposed staging
    // (the weights): rows kq*8 .. +7 of the chunk, columns cg*8 .. +7 of the
    // tile.  Direct staging (the activations): row m0 + 32 i (i = 0..7) of
    // the tile, k-group g of the chunk.
    const int op = wave >> 2;
    const bool direct = op == 0;
    const int cg = tid & 31, kq = (tid >> 5) & 7;
    // (direct: 8 consecutive lanes take 8 consecutive rows m0 of one k-group)
    const int m0_d = (tid & 7) | (((tid >> 6) & 3) << 3), g_d = (tid >> 3) & 7;
    constexpr int kRsrcWord3 = 0x00020000;
    __amdgpu_buffer_rsrc_t rs, rs1;
    uint32_t vo;
    int row_bytes;
        if (op == 0) {
            rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.A + (int64_t)m_base * p.lda), (short)0,
                                                   (int)((int64_t)rows_tile * p.lda * 2), kRsrcWord3);
            rs1 = rs;
            vo = (uint32_t)((m0_d * p.lda + g_d * 8) * 2);
            row_bytes = (int)(p.lda * 2);
        } else {
            const int col = n_base + cg * 8;
            const int64_t eoff = (int64_t)e * p.bstride;
            rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.B0 + eoff), (short)0,
                                                   (int)((int64_t)p.K1 * p.ldb * 2), kRsrcWord3);
            rs1 = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)(p.B1 ? p.B1 : p.B0) + eoff), (short)0,
                                                    p.B1 ? (int)((int64_t)(p.K - p.K1) * p.ldb * 2) : 0, kRsrcWord3);
            vo = col < p.N ? (uint32_t)((kq * 8 * p.ldb + col) * 2) : 0x80000000u;
            row_bytes = (int)(p.ldb * 2);
        }
    u32x4_t st[8];
    auto load_row = [&](int ch, int i) __attribute__((always_inline)) {
        if (direct) {
            st[i] = __builtin_bit_cast(u32x4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(rs, vo, i * 32 * row_bytes + ch * KC * 2, 0));
        } else if (ch * KC >= p.K1) {
            st[i] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs1, vo, (ch * KC - p.K1 + i) * row_bytes, 0));
        } else {
            st[i] = __builtin_bit_cast(u32x4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (ch * KC + i) * row_bytes, 0));
        }
    };
    // LDS layout of one operand in one buffer (32 KB), in MFMA fragment
    // order: the 16 bytes of tile row m, k-group g (k = 8 g .. 8 g + 7 of the
    // chunk) sit in the 1 KB block 2 (m >> 4) + (g >> 2) at 16-byte position
    //   16 (g & 3) + (m & 8) + ((m & 7) ^ ((m >> 3) & 7)).
    // A fragment read (16 rows from R0, one k-step) is then one block, and
    // each aligned group of 8 lanes reads one aligned 128 bytes; measured on
    // MI355X with SQ_LDS_BANK_CONFLICT this read has no bank conflict, nor
    // have the writes below, which put 8 consecutive lanes into 8 distinct
    // 16-byte slots of 128-byte lines.  (The earlier row-major swizzle
    // g ^ (m & 7) ^ ((m >> 3) & 7) cost 4 conflict cycles per fragment read.)
    //
    // Transposed writes: column j of the thread's 8 x 8 block is row
    // m = 8 cg + j, group kq: block 2 (cg >> 1) + (kq >> 2), position
    // 16 (kq & 3) + 8 (cg & 1) + (j ^ (cg & 7)).
    const uint32_t w_lane = (uint32_t)((2 * (cg >> 1) + (kq >> 2)) * 1024 + 256 * (kq & 3) + 128 * (cg & 1));
    const int w_x = cg & 7;
    // v_perm selectors: column j takes the low (j even) or high halves of
    // rows 2q and 2q + 1
    const uint32_t sel_lo = 0x05040100u, sel_hi = 0x07060302u;
    // Direct writes: row m = m0 + 32 j, group g: block 2 (m0 >> 4) + 4 j +
    // (g >> 2), position 16 (g & 3) + (m0 & 8) + ((m0 & 7) ^ x_j) with
    // x_j = ((m0 >> 3) & 3) | ((j & 1) << 2).
    const uint32_t d_lane = (uint32_t)((2 * (m0_d >> 4) + (g_d >> 2)) * 1024 + 256 * (g_d & 3) + 16 * (m0_d & 8));
    const int d_x = (m0_d & 7) ^ ((m0_d >> 3) & 3);
    auto put_col = [&](int buf, int j) __attribute__((always_inline)) {
        if (direct) {
            const uint32_t off = d_lane + (uint32_t)(j * 4096) + (uint32_t)((d_x ^ ((j & 1) << 2)) << 4);
            *(u32x4_t*)(lds + (size_t)(buf * 2) * OPB + off) = st[j];
            return;
        }
        const uint32_t sel = (j & 1) ? sel_hi : sel_lo;
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_perm(st[2 * q + 1][j >> 1], st[2 * q][j >> 1], sel);
        const uint32_t off = w_lane + (uint32_t)((j ^ w_x) << 4);
        *(u32x4_t*)(lds + (size_t)(buf * 2 + op) * OPB + off) = v;
    };
    // Fragment reads: lane l takes row R0 + (l & 15), group 4 ks + (l >> 4),
    // i.e. position 16 (l >> 4) + (l & 8) + ((l & 7) ^ (2 b | ((l >> 3) & 1)))
    // of block 2 (R0 >> 4) + ks, with b = (R0 >> 4) & 3 known at compile time
    // (the wave's row offsets are multiples of 64).  The four lane offsets are
    // formed once per chunk with the buffer base folded in.
    uint32_t rb[4];
    auto set_read_base = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
            rb[bb] = (uint32_t)(buf * 2 * OPB) +
                     (uint32_t)(16 * (16 * (lane >> 4) + (lane & 8) + ((lane & 7) ^ ((2 * bb) | ((lane >> 3) & 1)))));
    };
    // buffer b: rb holds b's base; the other buffer is rb ^ (2 OPB)
    auto frag = [&](int other, int opf, int ks, int blk) __attribute__((always_inline)) {
        const int B = (opf == 0 ? wm * 4 : wn * 8) + blk;
        const uint32_t r = rb[blk & 3];
        const uint32_t a = (other ? (r ^ (uint32_t)(2 * OPB)) : r) + (uint32_t)(opf * OPB + (2 * B + ks) * 1024);
        return *(const u32x4_t*)(lds + a);
    };
    floatx4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // B fragment of group q of the current chunk: k-step q >> 3, n-block
    // q & 7; groups 16.. are the next chunk's (the other buffer)
    auto bfrag = [&](int q) __attribute__((always_inline)) {
        return q < 16 ? frag(0, 1, q >> 3, q & 7) : frag(1, 1, 0, q - 16);
    };
    // prologue: chunk 0 into buffer 0, chunk 1 staged, chunk 0's first
    // A fragments and first two B fragments in registers
#pragma unroll
    for (int i = 0; i < 8; ++i) load_row(0, i);
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < 8; ++j) put_col(0, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_row(1, i);
    lds_barrier();
    set_read_base(0);
    u32x4_t fa0[4], fa1[4], fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fa0[j] = frag(0, 0, 0, j);
    fb[0] = bfrag(0);
    fb[1] = bfrag(1);
    // chunk ch (buffer b): 16 groups q of 4 MFMAs (k-step q >> 3, n-block
    // q & 7, against the wave's 4 m-blocks); the B fragment of group q + 2
    // is read during group q into slot (q + 2) % 4 (16 groups per chunk keep
    // the slots aligned from one chunk to the next).  Groups 0-1 write the
    // staged chunk ch+1 into buffer b^1, groups 2-5 issue the loads of chunk
    // ch+2, groups 4-7 read the second k-step's A fragments.  One barrier,
    // after group 13, when every read of buffer b has been issued: chunk
    // ch+1 is then visible, so groups 14-15 read its first fragments and the
    // next chunk starts without waiting; and buffer b is free for the writes
    // of the next chunk.
    for (int ch = 0; ch < nch; ++ch) {
        const int b = ch & 1;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int ks = q >> 3, i = q & 7;
            if (ks == 0) {
                if (i == 0) wait_vmcnt<0>();
                if (i < 2) {
#pragma unroll
                    for (int j = 4 * i; j < 4 * i + 4; ++j) put_col(b ^ 1, j);
                } else if (i < 6) {
                    load_row(ch + 2, 2 * (i - 2));
                    load_row(ch + 2, 2 * (i - 2) + 1);
                }
                if (i >= 4) fa1[i - 4] = frag(0, 0, 1, i - 4);
            } else if (i >= 6) {
                fa0[2 * (i - 6)] = frag(1, 0, 0, 2 * (i - 6));
                fa0[2 * (i - 6) + 1] = frag(1, 0, 0, 2 * (i - 6) + 1);
            }
            fb[(q + 2) % 4] = bfrag(q + 2);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[q % 4]),
                                                                    __builtin_bit_cast(bf16x8_t, ks ? fa1[j] : fa0[j]),
                                                                    acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 13) {
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        set_read_base(b ^ 1);
    }
    // lane holds C[m][n .. n+3] of block (n-block i, m-block j)
    uint16_t* Ce = (uint16_t*)p.C + (int64_t)m_base * p.ldc;
    const int64_t ldc = p.ldc;
    if (ldc % 8 == 0 && p.N % 8 == 0 && (((uintptr_t)Ce) & 15) == 0) {
        // through LDS, so every global store covers whole 128-byte lines (a
        // lane's direct 8-byte stores leave each instruction 32 bytes of 16
        // rows): each wave stages its 64 x 128 outputs in its own region
        // (padded rows: the 16 rows x 2 column groups of a half wave hit 32
        // distinct bank pairs) and stores 4 rows of 256 bytes per instruction
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();   // every wave is past its last fragment read
        asm volatile("" ::: "memory");
        uint8_t* reg = lds + wave * 64 * SPITCH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ml = j * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x2_t w;
                w[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                w[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(u32x2_t*)(reg + ml * SPITCH + (i * 16 + 4 * (lane >> 4)) * 2) = w;
            }
        }
        const int lr = lane >> 4, lc = lane & 15;
        const int n = n_base + wn * 128 + lc * 8;
#pragma unroll
        for (int r = 0; r < 64; r += 4) {
            const int mr = r + lr;
            const u32x4_t v = *(const u32x4_t*)(reg + mr * SPITCH + lc * 16);
            const int ml = wm * 64 + mr;
            if (ml < rows_tile && n < p.N) *(u32x4_t*)(Ce + (int64_t)ml * ldc + n) = v;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ml = wm * 64 + j * 16 + (lane & 15);
        if (ml >= rows_tile) continue;
        const int m = ml;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int n = n_base + wn * 128 + i * 16 + 4 * (lane >> 4);
            if (n >= p.N) continue;
            uint2 w;
            w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *(uint2*)(Ce + (int64_t)m * ldc + n) = w;
        }
    }
#endif
}

// Weight gradients, bf16, persistent: C_e = A_e^T B_e over the expert's
// rows, 256 x 256 tiles as in k_gemm_nn256 (same LDS layout, transposed
// staging and per-chunk schedule), but one block per CU walks its tiles as
// a single stream of 64-row chunks.  The loads two chunks ahead cross into
// the next tile, so a tile's first chunks arrive while the previous tile is
// still multiplying; at a tile's last chunk the block stages its outputs
// through the LDS buffer that chunk has just released (each wave its own
// 8 KB, 32 rows at a time), issues the stores and goes on with the next
// tile, whose first chunk is already in the other buffer.  The stores drain
// during the next tile's first chunk: the wait that ends that chunk's loads
// is taken before they are issued.  Experts with fewer rows than a tile
// need (or none) take one chunk that reads zeros.  Block b serves XCD b % 8;
// the 32 blocks of an XCD take consecutive tiles of that XCD's range, so
// concurrent tiles share an expert's rows in L2 as in the per-tile launch.
// The XCD ranges are contiguous and of equal cost, a tile costing its
// expert's 64-row chunks (at least one) plus kTileEnd for its output stores:
// a tile's time grows with its expert's rows, so ranges of equal tile counts
// left the XCD with the most rows (DeepSeek-V3: rows on 80 of 256 experts)
// finishing last.
__global__ __launch_bounds__(512) void k_gemm_wgrad(XnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BM = 256, KC = 64, GM = 4;
    constexpr int kTileEnd = 3;   // a tile's output stores, in chunk times (about 9000 against 3300 cycles)
    constexpr int OPB = BM * KC * 2;
    __shared__ __align__(16) uint8_t lds[4 * OPB];
    __shared__ int xcd_range[2];
    const int per_e = p.tiles_m * p.tiles_n;
    const int ntiles = p.E * per_e;
    const int xcd = blockIdx.x % 8, nslot = gridDim.x / 8;
    if (threadIdx.x < 64) {
        // wave 0: lane l sums the cost of experts [l s, l s + s), a wave scan
        // gives the cost before each segment, and for bound x (this XCD's
        // first tile and the next XCD's) the lane whose segment reaches
        // x total / 8 walks its experts to the first tile t with
        // 8 cost(tiles before t) >= x total
        const int l = threadIdx.x, seg = (p.E + 63) / 64;
        const int e0 = min(l * seg, p.E), e1 = min(e0 + seg, p.E);
        auto cost = [&](int e) -> int64_t {
            const int rows = p.offsets[e + 1] - p.offsets[e];
            return (int64_t)per_e * (max(1, (rows + KC - 1) / KC) + kTileEnd);
        };
        int64_t own = 0;
        for (int e = e0; e < e1; ++e) own += cost(e);
        int64_t inc = own;
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t v = __shfl_up(inc, o);
            if (l >= o) inc += v;
        }
        const int64_t total = __shfl(inc, 63);
        for (int j = 0; j < 2; ++j) {
            const int x = xcd + j;
            int t = x == 0 ? 0 : ntiles;
            if (x > 0 && x < 8) {
                const int64_t target = (int64_t)x * total;
                const uint64_t reach = __ballot(8 * inc >= target);
                const int src = __ffsll((unsigned long long)reach) - 1;
                int cand = e1 * per_e;
                int64_t c = inc - own;
                for (int e = e0; e < e1; ++e) {
                    const int64_t ce = cost(e);
                    if (8 * (c + ce) >= target) {
                        const int64_t per_tile = ce / per_e;
                        const int64_t need = target - 8 * c;
                        cand = e * per_e + (int)(need > 0 ? (need + 8 * per_tile - 1) / (8 * per_tile) : 0);
                        break;
                    }
                    c += ce;
                }
                t = __shfl(cand, src);
            }
            if (l == 0) xcd_range[j] = t;
        }
    }
    __syncthreads();
    const int t_end = xcd_range[1];
    const int t_first = xcd_range[0] + (int)(blockIdx.x / 8);
    if (t_first >= t_end) return;

    // tile -> expert and 256 x 256 block of C_e, in groups of GM row tiles
    // (the 32 CUs of an XCD run 4 row tiles x 8 column tiles at a time)
    int te, tmb, tnb, tlo, trows;
    auto decode = [&](int tile) __attribute__((always_inline)) {
        const int e = tile / per_e;
        const int L = tile - e * per_e;
        const int grp = L / (GM * p.tiles_n);
        const int gm = min(p.tiles_m - grp * GM, GM);
        const int in = L - grp * GM * p.tiles_n;
        te = __builtin_amdgcn_readfirstlane(e);
        tmb = __builtin_amdgcn_readfirstlane((grp * GM + in % gm) * BM);
        tnb = __builtin_amdgcn_readfirstlane((in / gm) * BM);
        tlo = __builtin_amdgcn_readfirstlane(p.offsets[te]);
        trows = __builtin_amdgcn_readfirstlane(p.offsets[te + 1]) - tlo;
    };
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // load cursor: operand op (0: A, 1: B) of this thread, rows kq*8 .. +7
    // of the chunk, columns cg*8 .. +7 of the tile
    const int op = wave >> 2;
    const int cg = tid & 31, kq = (tid >> 5) & 7;
    const uint16_t* src = (const uint16_t*)(op == 0 ? p.A : p.B0);
    const int64_t ld = op == 0 ? p.lda : p.ldb;
    const int lim = op == 0 ? p.M : p.N;
    const int row_bytes = (int)(ld * 2);
    constexpr int kRsrcWord3 = 0x00020000;
    int lt = t_first, lch = 0, lnch = 1;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t vo;
    auto load_setup = [&]() __attribute__((always_inline)) {
        decode(lt);
        lnch = max(1, (trows + KC - 1) / KC);
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + (int64_t)tlo * ld), (short)0,
                                               (int)((int64_t)trows * ld * 2), kRsrcWord3);
        const int col = (op == 0 ? tmb : tnb) + cg * 8;
        vo = col < lim ? (uint32_t)((kq * 8 * ld + col) * 2) : 0x80000000u;
    };
    auto advance_load = [&]() __attribute__((always_inline)) {
        if (++lch == lnch) {
            lch = 0;
            lt += nslot;
            if (lt < t_end) load_setup();
        }
    };
    u32x4_t st[8];
    auto load_row = [&](int i) __attribute__((always_inline)) {
        st[i] = __builtin_bit_cast(u32x4_t,
                                   __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (lch * KC + i) * row_bytes, 0));
    };
    // LDS layout and transposed writes as in k_gemm_nn256: the chunk of tile
    // row m, k-group g in block 2 (m >> 4) + (g >> 2) at 16-byte position
    // 16 (g & 3) + (m & 8) + ((m & 7) ^ ((m >> 3) & 7)).
    const uint32_t w_lane = (uint32_t)((2 * (cg >> 1) + (kq >> 2)) * 1024 + 256 * (kq & 3) + 128 * (cg & 1));
    const int w_x = cg & 7;
    const uint32_t sel_lo = 0x05040100u, sel_hi = 0x07060302u;
    auto put_col = [&](int buf, int j) __attribute__((always_inline)) {
        const uint32_t sel = (j & 1) ? sel_hi : sel_lo;
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_perm(st[2 * q + 1][j >> 1], st[2 * q][j >> 1], sel);
        *(u32x4_t*)(lds + (size_t)(buf * 2 + op) * OPB + w_lane + (uint32_t)((j ^ w_x) << 4)) = v;
    };
    uint32_t rb[4];
    auto set_read_base = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
            rb[bb] = (uint32_t)(buf * 2 * OPB) +
                     (uint32_t)(16 * (16 * (lane >> 4) + (lane & 8) + ((lane & 7) ^ ((2 * bb) | ((lane >> 3) & 1)))));
    };
    auto frag = [&](int other, int opf, int ks, int blk) __attribute__((always_inline)) {
        const int B = (opf == 0 ? wm * 4 : wn * 8) + blk;
        const uint32_t r = rb[blk & 3];
        const uint32_t a = (other ? (r ^ (uint32_t)(2 * OPB)) : r) + (uint32_t)(opf * OPB + (2 * B + ks) * 1024);
        return *(const u32x4_t*)(lds + a);
    };
    floatx4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto bfrag = [&](int q) __attribute__((always_inline)) {
        return q < 16 ? frag(0, 1, q >> 3, q & 7) : frag(1, 1, 0, q - 16);
    };

    // compute cursor: the tile whose chunks are being multiplied
    int ct = t_first, cch = 0;
    decode(ct);
    int ce = te, cmb = tmb, cnb = tnb, cnch = max(1, (trows + KC - 1) / KC);
    const bool staged = p.N % 8 == 0 && (((uintptr_t)p.C) & 15) == 0;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    // outputs of the compute tile; buffer b is free (its last reads ended at
    // the chunk's barrier) and holds 8 KB per wave: 32 rows of 256 bytes
    // with 16-byte column group c of row r at slot c ^ (r & 15)
    auto epilogue = [&](int b) __attribute__((always_inline)) {
        uint16_t* Ce = (uint16_t*)p.C + (size_t)ce * p.M * p.N;
        wait_vmcnt<0>();   // the loads of the chunk after next have landed before the stores join the count
        if (staged) {
            uint8_t* reg = lds + b * 2 * OPB + wave * 8192;
            const int lr = lane >> 4, lc = lane & 15;
            const int n = cnb + wn * 128 + lc * 8;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int ml = jj * 16 + lc;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int c = 2 * i + (lr >> 1);
                        u32x2_t w;
                        w[0] = pack_bf16x2(acc[i][2 * h + jj][0], acc[i][2 * h + jj][1]);
                        w[1] = pack_bf16x2(acc[i][2 * h + jj][2], acc[i][2 * h + jj][3]);
                        *(u32x2_t*)(reg + ml * 256 + ((c ^ lc) << 4) + (lr & 1) * 8) = w;
                    }
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int mr = 4 * r + lr;
                    const u32x4_t v = *(const u32x4_t*)(reg + mr * 256 + ((lc ^ (mr & 15)) << 4));
                    const int m = cmb + wm * 64 + h * 32 + mr;
                    if (m < p.M && n < p.N) *(u32x4_t*)(Ce + (int64_t)m * p.N + n) = v;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = cmb + wm * 64 + j * 16 + (lane & 15);
                if (m >= p.M) continue;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int n = cnb + wn * 128 + i * 16 + 4 * (lane >> 4);
                    if (n >= p.N) continue;
                    uint2 w;
                    w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                    w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                    *(uint2*)(Ce + (int64_t)m * p.N + n) = w;
                }
            }
        }
        lds_barrier();   // every wave is done with buffer b before it is refilled
    };

    // prologue: stream chunk 0 into buffer 0, chunk 1 staged in registers
    load_setup();
#pragma unroll
    for (int i = 0; i < 8; ++i) load_row(i);
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < 8; ++j) put_col(0, j);
    advance_load();
    if (lt < t_end) {
#pragma unroll
        for (int i = 0; i < 8; ++i) load_row(i);
    }
    advance_load();
    lds_barrier();
    set_read_base(0);
    u32x4_t fa0[4], fa1[4], fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fa0[j] = frag(0, 0, 0, j);
    fb[0] = bfrag(0);
    fb[1] = bfrag(1);
    // stream chunk s (buffer b = s & 1): the schedule of k_gemm_nn256, with
    // the loads of stream chunk s + 2 in groups 2-5; the load cursor moves on
    // at the end of the chunk
    bool fresh = false;   // the chunk before ended a tile and waited for the loads
    for (int s = 0;; ++s) {
        const int b = s & 1;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int ks = q >> 3, i = q & 7;
            if (ks == 0) {
                if (i == 0 && !fresh) wait_vmcnt<0>();
                if (i < 2) {
#pragma unroll
                    for (int j = 4 * i; j < 4 * i + 4; ++j) put_col(b ^ 1, j);
                } else if (i < 6) {
                    if (lt < t_end) {
                        load_row(2 * (i - 2));
                        load_row(2 * (i - 2) + 1);
                    }
                }
                if (i >= 4) fa1[i - 4] = frag(0, 0, 1, i - 4);
            } else if (i >= 6) {
                fa0[2 * (i - 6)] = frag(1, 0, 0, 2 * (i - 6));
                fa0[2 * (i - 6) + 1] = frag(1, 0, 0, 2 * (i - 6) + 1);
            }
            fb[(q + 2) % 4] = bfrag(q + 2);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[q % 4]),
                                                                    __builtin_bit_cast(bf16x8_t, ks ? fa1[j] : fa0[j]),
                                                                    acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 13) {
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        fresh = false;
        set_read_base(b ^ 1);
        advance_load();
        if (++cch == cnch) {
            epilogue(b);
            ct += nslot;
            if (ct >= t_end) break;
            decode(ct);
            ce = te; cmb = tmb; cnb = tnb; cnch = max(1, (trows + KC - 1) / KC);
            cch = 0;
            fresh = true;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
#endif
}

// Blocks of the persistent weight-gradient launch: the current device's CU
// count, rounded down to a multiple of 8 (at least 8), read once per device.
static int wgrad_blocks() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        cached[dev] = cus / 8 * 8;
    }
    return cached[dev];
}

hipError_t launch_gemm_tn(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int M, int N,
                          int E, const int32_t* offsets, int64_t max_rows, hipStream_t s) {
    // the 256 x 256 kernel addresses an expert's rows (plus two chunks of
    // read-ahead) with 32-bit buffer offsets
    const int64_t ldmax = lda > ldb ? lda : ldb;
    if (bf16 && M >= 256 && N >= 256 && (max_rows + 128) * ldmax * 2 < ((int64_t)1 << 31)) {
        XnParams p = {};
        p.A = A; p.lda = lda; p.B0 = B; p.ldb = ldb; p.C = C;
        p.M = M; p.N = N; p.E = E;
        p.tiles_m = (M + 255) / 256;
        p.tiles_n = (N + 255) / 256;
        p.offsets = offsets;
        const int64_t nt = (int64_t)E * p.tiles_m * p.tiles_n;
        if (nt <= 0) return hipSuccess;
        if (nt > 0x7fffffff - 8) return hipErrorInvalidValue;
        // one block per CU (128 KB of LDS each), a multiple of 8 blocks
        const int64_t grid = (nt + 7) / 8 * 8 < wgrad_blocks() ? (nt + 7) / 8 * 8 : wgrad_blocks();
        hipLaunchKernelGGL(k_gemm_wgrad, dim3((unsigned)grid), dim3(512), 0, s, p);
        return hipGetLastError();
    }
    TnParams p;
    p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.C = C;
    p.M = M; p.N = N; p.E = E;
    p.tiles_m = (M + 127) / 128;
    p.tiles_n = (N + 127) / 128;
    p.offsets = offsets;
    const int64_t grid = (int64_t)E * p.tiles_m * p.tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (bf16) hipLaunchKernelGGL(k_gemm_tn<true>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(k_gemm_tn<false>, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

__global__ void k_single_group(int32_t* offsets, int rows) {
    if (threadIdx.x == 0) {
        offsets[0] = 0;
        offsets[1] = rows;
    }
}

void launch_single_group_offsets(int32_t* offsets, int64_t rows, hipStream_t s) {
    hipLaunchKernelGGL(k_single_group, dim3(1), dim3(64), 0, s, offsets, (int)rows);
}

// Row-tile prefix of the NN product: prefix[e+1] = prefix[e] + ceil(rows_e / 256).
__global__ __launch_bounds__(1024) void k_nn_plan(const int32_t* __restrict__ offsets, int E,
                                                  int32_t* __restrict__ prefix) {
    __shared__ int32_t scan[1024];
    const int e = threadIdx.x;
    scan[e] = e < E ? (offsets[e + 1] - offsets[e] + 255) / 256 : 0;
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

bool gemm_nn_supported(int64_t max_rows, int64_t lda, int K, int K1, int64_t ldb, int N) {
    // 32-bit buffer offsets: a 256-row tile of A, and K1 / K - K1 rows of B
    // (plus two chunks of read-ahead)
    return N >= 256 && K % 64 == 0 && K1 % 64 == 0 && max_rows > 0 && 256 * lda * 2 < ((int64_t)1 << 31) &&
           ((int64_t)K + 128) * ldb * 2 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_nn(const void* A, int64_t lda, const void* B0, const void* B1, int K1, int64_t ldb,
                          int64_t bstride, void* C, int64_t ldc, int N, int K, int E, const int32_t* offsets,
                          int64_t max_rows, int32_t* prefix, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_nn_plan, dim3(1), dim3(1024), 0, s, offsets, E, prefix);
    XnParams p = {};
    p.A = A; p.lda = lda; p.B0 = B0; p.B1 = B1; p.ldb = ldb; p.bstride = bstride;
    p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.K1 = B1 ? K1 : K; p.E = E;
    p.tiles_n = (N + 255) / 256;
    p.offsets = offsets;
    p.prefix = prefix;
    const int64_t mt_ub = (max_rows + 255) / 256 + E;
    const int64_t nt = mt_ub * p.tiles_n;
    if (nt > 0x7fffffff - 8) return hipErrorInvalidValue;
    const int64_t grid = (nt + 7) / 8 * 8;
    hipLaunchKernelGGL(k_gemm_nn256, dim3((unsigned)grid), dim3(512), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router.  One wave per token: z_e = dots[t][e] (+ logit_bias[e]) exactly as
// the forward forms it, then dz by the gate family (see moe.h):
//   softmax over the selected:    dz_e = g_j (dg_j - sum_i g_i dg_i)  (e = idx_j)
//   full softmax / expert choice: dz = p (dp - <p, dp>), p = softmax(z)
//   sigmoid with selection bias:  dz_e = (dg_j - sum_i g_i dg_i) / S s_e (1 - s_e),
//                                 S = sum of s over the selected
// Slots of one token hold distinct experts, so dp_e is one dg; each dz
// element is written once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_router(const float* __restrict__ dots, int NC,
                                                    const float* __restrict__ logit_bias,
                                                    const int32_t* __restrict__ idx, const float* __restrict__ gates,
                                                    const float* __restrict__ dg, int gate, int T, int E, int slots,
                                                    float* __restrict__ dz) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + w;
    if (t >= T) return;
    const int32_t* it = idx + (int64_t)t * slots;
    const float* gt = gates + (int64_t)t * slots;
    const float* dgt = dg + (int64_t)t * slots;
    float* dzt = dz + (int64_t)t * E;
    auto zv = [&](int e) { return logit_bias ? dots[(int64_t)t * NC + e] + logit_bias[e] : dots[(int64_t)t * NC + e]; };
    auto wsum = [&](float v) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        return v;
    };
    // slot of expert e in this token's selection, or -1 (expert choice keeps
    // slot e for expert e)
    auto slot_of = [&](int e) {
        if (gate == MOE_GATE_EXPERT_CHOICE) return it[e] >= 0 ? e : -1;
        for (int j = 0; j < slots; ++j)
            if (it[j] == e) return j;
        return -1;
    };
    if (gate == MOE_GATE_SOFTMAX_FULL || gate == MOE_GATE_EXPERT_CHOICE) {
        float m = -INFINITY;
        for (int e = lane; e < E; e += 64) m = fmaxf(m, zv(e));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        float sum = 0.0f;
        for (int e = lane; e < E; e += 64) sum += canon::expc(zv(e) - m);
        sum = wsum(sum);
        float c = 0.0f;
        for (int e = lane; e < E; e += 64) {
            const int j = slot_of(e);
            if (j >= 0) c += canon::expc(zv(e) - m) / sum * dgt[j];
        }
        c = wsum(c);
        for (int e = lane; e < E; e += 64) {
            const int j = slot_of(e);
            const float pe = canon::expc(zv(e) - m) / sum;
            dzt[e] = pe * ((j >= 0 ? dgt[j] : 0.0f) - c);
        }
        return;
    }
    // selected-slot families: c = sum_j g_j dg_j over the token's slots
    float c = 0.0f, S = 0.0f;
    for (int j = lane; j < slots; j += 64) {
        if (it[j] >= 0) {
            c += gt[j] * dgt[j];
            if (gate == MOE_GATE_SIGMOID_BIAS) S += canon::sigmoidc(zv(it[j]));
        }
    }
    c = wsum(c);
    S = wsum(S);
    for (int e = lane; e < E; e += 64) {
        const int j = slot_of(e);
        float v = 0.0f;
        if (j >= 0) {
            if (gate == MOE_GATE_SIGMOID_BIAS) {
                const float s = canon::sigmoidc(zv(e));
                v = (dgt[j] - c) / S * (s * (1.0f - s));
            } else {
                v = gt[j] * (dgt[j] - c);
            }
        }
        dzt[e] = v;
    }
}

void launch_bwd_router(const float* dots, int NC, const float* logit_bias, const int32_t* idx, const float* gates,
                       const float* dg, int gate, int T, int E, int slots, float* dz, hipStream_t s) {
    if (T <= 0) return;
    hipLaunchKernelGGL(k_bwd_router, dim3((T + 3) / 4), dim3(256), 0, s, dots, NC, logit_bias, idx, gates, dg, gate,
                       T, E, slots, dz);
}

// Token gradient, one block per token, fp32 in this order: residual dY,
// routed rows in slot order, shared expert, then the router term dz_t W_r:
// over the token's selected experts in slot order when dz is zero elsewhere
// (idx != NULL: softmax over the selected, sigmoid), else over all experts
// in ascending order.
template <bool BF16>
__global__ __launch_bounds__(256) void k_bwd_dx(const void* __restrict__ dy, const void* __restrict__ dx_perm,
                                                const int32_t* __restrict__ slot_pos, int slots,
                                                const void* __restrict__ dx_shared, const float* __restrict__ dz,
                                                const int32_t* __restrict__ idx, const float* __restrict__ w_router,
                                                int E, int d, bool residual, void* __restrict__ dx) {
    const int t = blockIdx.x;
    const int32_t* sp = slot_pos + (int64_t)t * slots;
    const int32_t* it = idx ? idx + (int64_t)t * slots : nullptr;
    const float* dzt = dz ? dz + (int64_t)t * E : nullptr;
    if (d % 8 == 0 && ((((uintptr_t)dy) | ((uintptr_t)dx_perm) | ((uintptr_t)dx_shared) | ((uintptr_t)w_router) |
                        ((uintptr_t)dx)) & 15) == 0) {
        // 8 consecutive columns per thread and step (16-byte accesses); the
        // same operations per element in the same order as below
        for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
            float v[8], q[8];
            if (residual) load8<BF16>(dy, (int64_t)t * d + c, v);
            else {
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = 0.0f;
            }
            for (int j = 0; j < slots; ++j) {
                const int r = sp[j];
                if (r >= 0) {
                    load8<BF16>(dx_perm, (int64_t)r * d + c, q);
#pragma unroll
                    for (int u = 0; u < 8; ++u) v[u] += q[u];
                }
            }
            if (dx_shared) {
                load8<BF16>(dx_shared, (int64_t)t * d + c, q);
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] += q[u];
            }
            auto add_router = [&](int e) {
                load8<false>(w_router, (int64_t)e * d + c, q);
                const float z = dzt[e];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] += z * q[u];
            };
            if (dzt && it) {
                for (int j = 0; j < slots; ++j) {
                    const int e = it[j];
                    if (e >= 0) add_router(e);
                }
            } else if (dzt) {
                for (int e = 0; e < E; ++e) add_router(e);
            }
            store8<BF16>(dx, (int64_t)t * d + c, v);
        }
        return;
    }
    for (int c = threadIdx.x; c < d; c += 256) {
        float v = residual ? load_act<BF16>(dy, (int64_t)t * d + c) : 0.0f;
        for (int j = 0; j < slots; ++j) {
            const int r = sp[j];
            if (r >= 0) v += load_act<BF16>(dx_perm, (int64_t)r * d + c);
        }
        if (dx_shared) v += load_act<BF16>(dx_shared, (int64_t)t * d + c);
        if (dzt && it) {
            for (int j = 0; j < slots; ++j) {
                const int e = it[j];
                if (e >= 0) v += dzt[e] * w_router[(int64_t)e * d + c];
            }
        } else if (dzt) {
            for (int e = 0; e < E; ++e) v += dzt[e] * w_router[(int64_t)e * d + c];
        }
        store_act<BF16>(dx, (int64_t)t * d + c, v);
    }
}

void launch_bwd_dx(bool bf16, const void* dy, const void* dx_perm, const int32_t* slot_pos, int slots,
                   const void* dx_shared, const float* dz, const int32_t* idx, const float* w_router, int T, int E,
                   int d, bool residual, void* dx, hipStream_t s) {
    if (T <= 0) return;
    if (bf16)
        hipLaunchKernelGGL(k_bwd_dx<true>, dim3(T), dim3(256), 0, s, dy, dx_perm, slot_pos, slots, dx_shared, dz,
                           idx, w_router, E, d, residual, dx);
    else
        hipLaunchKernelGGL(k_bwd_dx<false>, dim3(T), dim3(256), 0, s, dy, dx_perm, slot_pos, slots, dx_shared, dz,
                           idx, w_router, E, d, residual, dx);
}

// Router gradients dW_r = dz^T x and db = sum_t dz, in two fixed-order
// passes: partial sums per token chunk, then k_bwd_wr_sum adds the chunks in
// order.  Column d of a partial row is the bias (x read as 1 there).
// More than 16 experts (k_bwd_wr_mma): chunks of 512 tokens on the fp32
// matrix cores, blocks of 64 experts x 256 columns.
constexpr int kWrTokens = 512;
// Up to 16 experts (k_bwd_wr_few): 32-token chunks, each thread 8 columns
// (one 16-byte load of bf16 x per token, or two of fp32) and every expert of
// the call, so no multiply-add is spent on absent experts and x is read once.
constexpr int kWrFewTokens = 32;
constexpr int kWrFewExperts = 16;

int bwd_wr_chunks(int T, int E) {
    const int tok = E <= kWrFewExperts ? kWrFewTokens : kWrTokens;
    return (T + tok - 1) / tok;
}

template <int EX, bool BF16>
__global__ __launch_bounds__(256) void k_bwd_wr_few(const float* __restrict__ dz, const void* __restrict__ x, int T,
                                                    int E, int d, float* __restrict__ part) {
    constexpr int CPT = 8;    // columns per thread
    __shared__ float zs[kWrFewTokens][EX];
    const int q = blockIdx.z;
    const int c0 = (blockIdx.x * 256 + threadIdx.x) * CPT;
    const int t0 = q * kWrFewTokens, nt = min(T - t0, kWrFewTokens);
    for (int i = threadIdx.x; i < kWrFewTokens * EX; i += 256) {
        const int tt = i / EX, ee = i - tt * EX;
        zs[tt][ee] = (tt < nt && ee < E) ? dz[(int64_t)(t0 + tt) * E + ee] : 0.0f;
    }
    __syncthreads();
    if (c0 > d) return;
    float acc[EX][CPT];
#pragma unroll
    for (int ee = 0; ee < EX; ++ee)
#pragma unroll
        for (int u = 0; u < CPT; ++u) acc[ee][u] = 0.0f;
    // whole vector loads where all 8 columns are below d (x rows 16-byte
    // aligned), else per column; column d itself is the bias (x = 1)
    const bool vec = c0 + CPT <= d && (d % CPT) == 0;
    auto row = [&](int tt, float* xv) {
        const int64_t base = (int64_t)(t0 + tt) * d + c0;
        if (vec) {
            if constexpr (BF16) {
                const u32x4_t v = *(const u32x4_t*)((const uint16_t*)x + base);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xv[2 * h] = __uint_as_float(v[h] << 16);
                    xv[2 * h + 1] = __uint_as_float(v[h] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4*)((const float*)x + base), b = *(const float4*)((const float*)x + base + 4);
                xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
                xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int c = c0 + u;
                xv[u] = c < d ? load_act<BF16>(x, base + u) : (c == d ? 1.0f : 0.0f);
            }
        }
    };
    constexpr int UT = 8;     // tokens whose rows are loaded before their multiply-adds
    for (int tb = 0; tb < nt; tb += UT) {
        float xv[UT][CPT];
#pragma unroll
        for (int j = 0; j < UT; ++j) {
            if (tb + j < nt) row(tb + j, xv[j]);
            else {
#pragma unroll
                for (int u = 0; u < CPT; ++u) xv[j][u] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < UT; ++j) {
            // past the chunk's tokens the rows are zero and zs reads 0: the
            // multiply-adds add +0 and change nothing, so they are not skipped
            const int tj = min(tb + j, kWrFewTokens - 1);
#pragma unroll
            for (int ee = 0; ee < EX; ++ee) {
                const float z = tb + j < nt ? zs[tj][ee] : 0.0f;
#pragma unroll
                for (int u = 0; u < CPT; ++u) acc[ee][u] += z * xv[j][u];
            }
        }
    }
#pragma unroll
    for (int ee = 0; ee < EX; ++ee) {
        if (ee < E) {
            float* dst = part + ((int64_t)q * E + ee) * (d + 1);
#pragma unroll
            for (int u = 0; u < CPT; ++u)
                if (c0 + u <= d) dst[c0 + u] = acc[ee][u];
        }
    }
}

// part[q][e][c] = sum over the tokens t of chunk q of dz[t][e] x[t][c], c <= d
// (x[t][d] = 1), with v_mfma_f32_16x16x4_f32: at k-step s a lane supplies
// token t0 + 4 s + (lane >> 4), expert e0 + 16 eb + (lane & 15) for block row
// eb and column c0 + 16 cb + (lane & 15) for block column cb; the wave's
// 4 x 4 blocks cover 64 experts x 64 columns, the block's 4 waves 256
// columns.  Each output lands on a lane as C[4 (lane >> 4) + i][lane & 15],
// so a store covers 4 rows of 64 contiguous bytes.  Tokens are added in
// k-step order, four per MFMA, so the partials do not depend on the launch.
template <bool BF16>
__global__ __launch_bounds__(256) void k_bwd_wr_mma(const float* __restrict__ dz, const void* __restrict__ x, int T,
                                                    int E, int d, float* __restrict__ part) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int KG = 4;   // k-steps per loop turn (16 tokens)
    const int e0 = blockIdx.x * 64, q = blockIdx.z;
    const int lane = threadIdx.x & 63, r = lane & 15, kk = lane >> 4;
    const int c0 = blockIdx.y * 256 + (threadIdx.x >> 6) * 64;
    const int t0 = q * kWrTokens, nt = min(T - t0, kWrTokens);
    // loads through buffer descriptors over the chunk's rows: experts past E,
    // columns past d - 1 and tokens past the chunk read zeros; the bias
    // column d adds 1 for each token of the chunk
    constexpr int kRsrcWord3 = 0x00020000;
    constexpr int XB = BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(dz + (int64_t)t0 * E), (short)0, nt * E * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)x + (int64_t)t0 * d * XB), (short)0, nt * d * XB, kRsrcWord3);
    uint32_t zo[4], xo[4];
    float c1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = e0 + 16 * u + r, c = c0 + 16 * u + r;
        zo[u] = e < E ? (uint32_t)((kk * E + e) * 4) : 0x80000000u;
        xo[u] = c < d ? (uint32_t)((kk * d + c) * XB) : 0x80000000u;
        c1[u] = c == d ? 1.0f : 0.0f;
    }
    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float fa0[KG][4], fb0[KG][4], fa1[KG][4], fb1[KG][4];
    auto load = [&](float (&fa)[KG][4], float (&fb)[KG][4], int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < KG; ++g) {
            const int tk = 4 * (s0 + g);   // first token of the k-step in the chunk
            const bool tv = tk + kk < nt;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                fa[g][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, zo[u], tk * E * 4, 0));
                float xv;
                if constexpr (BF16)
                    xv = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, xo[u], tk * d * 2, 0)
                                         << 16);
                else
                    xv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, xo[u], tk * d * 4, 0));
                fb[g][u] = xv + (tv ? c1[u] : 0.0f);
            }
        }
    };
    auto mma = [&](const float (&fa)[KG][4], const float (&fb)[KG][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[g][i], fb[g][j], acc[i][j], 0, 0, 0);
    };
    // k-steps past the chunk hold zeros; the next KG k-steps load during the
    // current ones
    const int nsteps = (nt + 3) / 4;
    load(fa0, fb0, 0);
    for (int s0 = 0; s0 < nsteps; s0 += 2 * KG) {
        if (s0 + KG < nsteps) load(fa1, fb1, s0 + KG);
        mma(fa0, fb0);
        if (s0 + KG >= nsteps) break;
        if (s0 + 2 * KG < nsteps) load(fa0, fb0, s0 + 2 * KG);
        mma(fa1, fb1);
    }
    float* pq = part + (int64_t)q * E * (d + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int e = e0 + 16 * i + 4 * kk + v;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = c0 + 16 * j + r;
                if (e < E && c <= d) pq[(int64_t)e * (d + 1) + c] = acc[i][j][v];
            }
        }
#endif
}

__global__ __launch_bounds__(256) void k_bwd_wr_sum(const float* __restrict__ part, int nq, int E, int d,
                                                    float* __restrict__ dw, float* __restrict__ db) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)E * (d + 1);
    if (i >= n) return;
    // chunks in order; 8 loads in flight ahead of the ordered adds
    float v = 0.0f;
    int q = 0;
    for (; q + 8 <= nq; q += 8) {
        float h[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = part[(int64_t)(q + u) * n + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += h[u];
    }
    for (; q < nq; ++q) v += part[(int64_t)q * n + i];
    const int e = (int)(i / (d + 1)), c = (int)(i - (int64_t)e * (d + 1));
    if (c < d) {
        if (dw) dw[(int64_t)e * d + c] = v;
    } else if (db) {
        db[e] = v;
    }
}

void launch_bwd_wr(bool bf16, const float* dz, const void* x, int T, int E, int d, float* part, float* dw, float* db,
                   hipStream_t s) {
    const int nq = bwd_wr_chunks(T, E);
    if (nq > 0 && E <= kWrFewExperts) {
        const dim3 grid((d + 1 + 256 * 8 - 1) / (256 * 8), 1, nq);
        if (E <= 8) {
            if (bf16) hipLaunchKernelGGL((k_bwd_wr_few<8, true>), grid, dim3(256), 0, s, dz, x, T, E, d, part);
            else hipLaunchKernelGGL((k_bwd_wr_few<8, false>), grid, dim3(256), 0, s, dz, x, T, E, d, part);
        } else {
            if (bf16) hipLaunchKernelGGL((k_bwd_wr_few<16, true>), grid, dim3(256), 0, s, dz, x, T, E, d, part);
            else hipLaunchKernelGGL((k_bwd_wr_few<16, false>), grid, dim3(256), 0, s, dz, x, T, E, d, part);
        }
    } else if (nq > 0) {
        const dim3 grid((E + 63) / 64, (d + 1 + 255) / 256, nq);
        if (bf16) hipLaunchKernelGGL(k_bwd_wr_mma<true>, grid, dim3(256), 0, s, dz, x, T, E, d, part);
        else hipLaunchKernelGGL(k_bwd_wr_mma<false>, grid, dim3(256), 0, s, dz, x, T, E, d, part);
    }
    const int64_t n = (int64_t)E * (d + 1);
    hipLaunchKernelGGL(k_bwd_wr_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, nq, E, d, dw, db);
}

}  // namespace moe
