// Combine stage for gfx950: gather each token's expert outputs back into token
// order and mix them with the gates,
//   out[t] = residual[t] + shared[t] + sum_j gate[t][j] * y_perm[slot_pos[t][j]]
// (CS25 "Lecture29" notes, eq. y = sum_i g_i(x) Expert_i(x); CS336 lecture 4
// notes, section 5 listing adds the residual; a dropped slot has
// slot_pos = -1 and contributes nothing, section 10).
//
// Gather form: one writer per output element and a fixed fp32 order
// (residual + shared first, then one fma per slot in slot order), so the
// result is bitwise reproducible without atomics.  Every thread moves 16-byte
// chunks; a block covers one or more whole tokens, so the token's slot rows
// and gates are block-uniform loads.
#include "device_common.h"
#include "kernels.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y_perm, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ gates, const void* __restrict__ residual,
                                                 const void* __restrict__ shared, void* __restrict__ out, int T,
                                                 int cpr, int k, int tpb) {
    constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    const int sub = threadIdx.x / (256 / tpb);           // token inside the block
    const int lt = threadIdx.x % (256 / tpb);            // thread inside the token
    const int t = blockIdx.x * tpb + sub;
    if (t >= T) return;
    const int tpt = 256 / tpb;
    for (int c = lt; c < cpr; c += tpt) {
        float acc[VEC];
        const int64_t off = (int64_t)t * cpr + c;
        if (residual) {
            const uint4 r = ((const uint4*)residual)[off];
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                acc[q] = BF16 ? bf16_bits_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu) : __uint_as_float(w[q]);
        } else {
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[q] = 0.0f;
        }
        if (shared) {
            const uint4 r = ((const uint4*)shared)[off];
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                acc[q] = acc[q] + (BF16 ? bf16_bits_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu) : __uint_as_float(w[q]));
        }
        for (int j = 0; j < k; ++j) {
            const int32_t row = slot_pos[(int64_t)t * k + j];
            if (row < 0) continue;
            const float g = gates[(int64_t)t * k + j];
            const uint4 r = ((const uint4*)y_perm)[(int64_t)row * cpr + c];
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                const float y = BF16 ? bf16_bits_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu) : __uint_as_float(w[q]);
                acc[q] = __builtin_fmaf(g, y, acc[q]);
            }
        }
        uint4 o;
        if constexpr (BF16) {
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
        } else {
            o.x = __float_as_uint(acc[0]); o.y = __float_as_uint(acc[1]);
            o.z = __float_as_uint(acc[2]); o.w = __float_as_uint(acc[3]);
        }
        ((uint4*)out)[off] = o;
    }
}

void launch_combine(const void* y_perm, const int32_t* slot_pos, const float* gates, const void* residual,
                    const void* shared, void* out, int T, int d, int k, bool bf16, hipStream_t s) {
    if (T <= 0) return;
    const int cpr = d * (bf16 ? 2 : 4) / 16;
    int tpb = 1;                       // tokens per block: fill 256 threads when rows are short
    while (tpb < 256 && cpr * tpb * 2 <= 256) tpb *= 2;
    const int nb = (T + tpb - 1) / tpb;
    if (bf16)
        hipLaunchKernelGGL(k_combine<true>, dim3(nb), dim3(256), 0, s, y_perm, slot_pos, gates, residual, shared, out,
                           T, cpr, k, tpb);
    else
        hipLaunchKernelGGL(k_combine<false>, dim3(nb), dim3(256), 0, s, y_perm, slot_pos, gates, residual, shared, out,
                           T, cpr, k, tpb);
}

}  // namespace moe
