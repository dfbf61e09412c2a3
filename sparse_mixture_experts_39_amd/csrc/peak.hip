// Achievable-peak microbenchmarks of one MI355X (gfx950), used by the
// benchmark to quote measured ceilings beside the published ones:
//   * matrix-core rate: waves issuing independent bf16 MFMAs back to back
//     from registers (no memory traffic), for the two bf16 shapes the
//     grouped GEMMs could use (16x16x32 and 32x32x16);
//   * device-memory copy rate: 16-byte loads and stores over buffers far
//     larger than the 256 MB last-level cache;
//   * a cache flush: a read pass over a buffer larger than the 256 MB
//     last-level cache, so that a timed stage finds neither its inputs nor
//     dirty lines of the previous stage in it.
// These entry points are a measurement aid and not part of the layer's ABI
// (include/moe.h); they are built into their own library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace {

using moe::bf16x8_t;
using moe::floatx16_t;
using moe::floatx4_t;

// Each wave computes a 128 x 128 tile of accumulators in the grouped GEMM's
// register pattern: NB weight fragments times NB activation fragments per
// k-step, weight fragment outer (64 16x16x32 blocks, or 16 32x32x16 blocks,
// 256 accumulator registers either way), iters k-steps of 128 x 128 x K
// (K = 32 or 16), i.e. iters * 1048576 (shape 16) or iters * 524288 (shape
// 32) flops per wave.  Operands are fixed per lane but differ between
// fragments and lanes (bit patterns of ordinary bf16 numbers), so the
// multipliers toggle as they do on real data.  The accumulator sum is stored
// so that nothing is optimised away.
template <int SHAPE>
__global__ __launch_bounds__(256) void k_peak_mfma(int iters, float* __restrict__ out) {
    constexpr int NB = SHAPE == 16 ? 8 : 4;
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 2654435761u;
    bf16x8_t a[NB], b[NB];
#pragma unroll
    for (int v = 0; v < NB; ++v) {
        moe::u32x4_t wa, wb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // bf16 pairs with exponents near 1.0 and random mantissas and signs
            const uint32_t r1 = (seed ^ (0x9e3779b9u * (4 * v + i + 1))) * 0x85ebca6bu;
            const uint32_t r2 = (seed ^ (0xc2b2ae35u * (4 * v + i + 7))) * 0x27d4eb2fu;
            wa[i] = (0x3f003f00u | (r1 & 0x807f807fu));
            wb[i] = (0x3f003f00u | (r2 & 0x807f807fu));
        }
        a[v] = __builtin_bit_cast(bf16x8_t, wa);
        b[v] = __builtin_bit_cast(bf16x8_t, wb);
    }
    float s = 0.0f;
    if constexpr (SHAPE == 16) {
        floatx4_t acc[NB][NB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[i], a[j], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    } else {
        floatx16_t acc[NB][NB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[i], a[j], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// dst[i] = src[i] for n16 16-byte chunks; each thread moves U chunks per
// round, a grid stride apart, with the U loads in flight together (NT:
// non-temporal loads and stores, which do not keep the lines in the caches).
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_peak_copy(const moe::u32x4_t* __restrict__ src, moe::u32x4_t* __restrict__ dst,
                                                   int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        moe::u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(&src[i + u * stride]) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (NT) __builtin_nontemporal_store(v[u], &dst[i + u * stride]);
            else dst[i + u * stride] = v[u];
        }
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

// A read pass over n16 16-byte chunks of buf: the lines it brings in evict
// whatever the caches held (a dirty line of an earlier kernel is written back
// here, not during the next timed kernel).  The chunks are folded into one
// word per thread that is stored only if it equals `never`, which keeps the
// loads from being optimised away.
__global__ __launch_bounds__(256) void k_touch16(const moe::u32x4_t* __restrict__ buf, int64_t n16, uint32_t never,
                                                 uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const moe::u32x4_t v = buf[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == never) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// MFMA rate probe: `blocks` blocks of 256 threads (4 waves), each wave
// issuing iters * 64 v_mfma_f32_16x16x32_bf16 (shape 16: iters * 1048576
// flops) or iters * 16 v_mfma_f32_32x32x16_bf16 (shape 32: iters * 524288
// flops).  out: blocks * 256 floats (device).  0 on success, -1 for
// bad arguments, else the HIP error.
int moe_peak_mfma(int shape, int iters, int blocks, float* out, void* stream) {
    if ((shape != 16 && shape != 32) || iters <= 0 || blocks <= 0 || !out) return -1;
    hipStream_t s = (hipStream_t)stream;
    if (shape == 16)
        hipLaunchKernelGGL(k_peak_mfma<16>, dim3(blocks), dim3(256), 0, s, iters, out);
    else
        hipLaunchKernelGGL(k_peak_mfma<32>, dim3(blocks), dim3(256), 0, s, iters, out);
    return (int)hipGetLastError();
}

// Copy probe: bytes (a multiple of 16) from src to dst, both device buffers
// of at least that size; `blocks` blocks of 256 threads, `unroll` (4 or 8)
// 16-byte chunks in flight per thread, non-temporal accesses when nt != 0.
int moe_peak_copy(const void* src, void* dst, int64_t bytes, int blocks, int unroll, int nt, void* stream) {
    if (!src || !dst || bytes <= 0 || (bytes & 15) || blocks <= 0 || (unroll != 4 && unroll != 8)) return -1;
    hipStream_t s = (hipStream_t)stream;
    const moe::u32x4_t* a = (const moe::u32x4_t*)src;
    moe::u32x4_t* b = (moe::u32x4_t*)dst;
    const int64_t n = bytes / 16;
    if (unroll == 4) {
        if (nt) hipLaunchKernelGGL((k_peak_copy<4, true>), dim3(blocks), dim3(256), 0, s, a, b, n);
        else hipLaunchKernelGGL((k_peak_copy<4, false>), dim3(blocks), dim3(256), 0, s, a, b, n);
    } else {
        if (nt) hipLaunchKernelGGL((k_peak_copy<8, true>), dim3(blocks), dim3(256), 0, s, a, b, n);
        else hipLaunchKernelGGL((k_peak_copy<8, false>), dim3(blocks), dim3(256), 0, s, a, b, n);
    }
    return (int)hipGetLastError();
}

// Cache flush: a read pass over `bytes` (a multiple of 16) of buf, a device
// buffer larger than the last-level cache; sink: 4096 * 256 uint32 of device
// memory that is written only in the (practically impossible) case that a
// thread's fold of its chunks equals `never`.
int moe_cache_flush(const void* buf, int64_t bytes, uint32_t never, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes <= 0 || (bytes & 15)) return -1;
    hipLaunchKernelGGL(k_touch16, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const moe::u32x4_t*)buf, bytes / 16,
                       never, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
