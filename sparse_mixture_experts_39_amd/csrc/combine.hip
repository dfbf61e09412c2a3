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
// chunks, several at once; a block covers whole tokens (or one token's chunk
// range for very wide rows), whose slot rows and gates it stages in LDS.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// The block owns tpb consecutive tokens and, of each of their rows, the
// chunks [c0, c0 + cw); its tpb * cw 16-byte output chunks go to its threads
// kCombU at a time (chunk q = tid + 256 u), so a thread keeps several
// expert-row loads in flight.  The tokens' slot rows and gates are staged in
// LDS when they fit.  Every output chunk is accumulated in the same order as
// always: residual + shared, then one fma per slot in slot order.
constexpr int kCombU = 8;           // output chunks per thread
constexpr int kCombMaxSlots = 512;  // slot entries staged per block

template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& r, float* out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    constexpr int VEC = BF16 ? 8 : 4;
#pragma unroll
    for (int q = 0; q < VEC; ++q)
        out[q] = BF16 ? bf16_bits_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu) : __uint_as_float(w[q]);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y_perm, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ gates, const void* __restrict__ residual,
                                                 const void* __restrict__ shared, void* __restrict__ out, int T,
                                                 int cpr, int k, int tpb, int c0, int cw) {
    constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    __shared__ int32_t srow[kCombMaxSlots];
    __shared__ float sg[kCombMaxSlots];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int nt = (int)min((int64_t)tpb, (int64_t)T - t0);
    if (nt <= 0) return;
    const bool staged = nt * k <= kCombMaxSlots;     // block-uniform
    if (staged) {
        for (int i = tid; i < nt * k; i += 256) {
            srow[i] = slot_pos[t0 * k + i];
            sg[i] = gates[t0 * k + i];
        }
        __syncthreads();
    }
    auto row_of = [&](int tl, int j) { return staged ? srow[tl * k + j] : slot_pos[(t0 + tl) * k + j]; };
    auto gate_of = [&](int tl, int j) { return staged ? sg[tl * k + j] : gates[(t0 + tl) * k + j]; };
    const int nch = nt * cw;
    const uint4* yp = (const uint4*)y_perm;
#pragma unroll
    for (int u0 = 0; u0 < kCombU; u0 += 4) {
        float acc[4][VEC];
        int tl[4], col[4];
        bool live[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + 256 * (u0 + u);
            live[u] = q < nch;
            tl[u] = live[u] ? q / cw : 0;
            col[u] = c0 + (q - tl[u] * cw);
            const int64_t off = (t0 + tl[u]) * cpr + col[u];
            if (live[u] && residual) {
                unpack16<BF16>(((const uint4*)residual)[off], acc[u]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[u][e] = 0.0f;
            }
            if (live[u] && shared) {
                float sh[VEC];
                unpack16<BF16>(((const uint4*)shared)[off], sh);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[u][e] = acc[u][e] + sh[e];
            }
        }
        for (int j = 0; j < k; ++j) {
            uint4 r[4];
            float g[4];
            bool use[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t row = live[u] ? row_of(tl[u], j) : -1;
                use[u] = row >= 0;       // a dropped slot contributes nothing
                g[u] = use[u] ? gate_of(tl[u], j) : 0.0f;
                if (use[u]) r[u] = yp[(int64_t)row * cpr + col[u]];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!use[u]) continue;
                float y[VEC];
                unpack16<BF16>(r[u], y);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[u][e] = __builtin_fmaf(g[u], y[e], acc[u][e]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (!live[u]) continue;
            uint4 o;
            if constexpr (BF16) {
                o.x = pack_bf16x2(acc[u][0], acc[u][1]);
                o.y = pack_bf16x2(acc[u][2], acc[u][3]);
                o.z = pack_bf16x2(acc[u][4], acc[u][5]);
                o.w = pack_bf16x2(acc[u][6], acc[u][7]);
            } else {
                o.x = __float_as_uint(acc[u][0]); o.y = __float_as_uint(acc[u][1]);
                o.z = __float_as_uint(acc[u][2]); o.w = __float_as_uint(acc[u][3]);
            }
            ((uint4*)out)[(t0 + tl[u]) * cpr + col[u]] = o;
        }
    }
}

void launch_combine(const void* y_perm, const int32_t* slot_pos, const float* gates, const void* residual,
                    const void* shared, void* out, int T, int d, int k, bool bf16, hipStream_t s) {
    if (T <= 0) return;
    const int cpr = d * (bf16 ? 2 : 4) / 16;
    constexpr int per_block = 256 * kCombU;
    // a row wider than one block's chunks is covered in column passes of
    // one token per block; otherwise a block takes as many whole rows as fit
    const int cw = cpr < per_block ? cpr : per_block;
    int tpb = per_block / cw;
    if (tpb * k > kCombMaxSlots) tpb = kCombMaxSlots / k > 0 ? kCombMaxSlots / k : 1;
    const int64_t nb = ((int64_t)T + tpb - 1) / tpb;
    for (int c0 = 0; c0 < cpr; c0 += cw) {
        const int w = cpr - c0 < cw ? cpr - c0 : cw;
        if (bf16)
            hipLaunchKernelGGL(k_combine<true>, dim3((unsigned)nb), dim3(256), 0, s, y_perm, slot_pos, gates,
                               residual, shared, out, T, cpr, k, tpb, c0, w);
        else
            hipLaunchKernelGGL(k_combine<false>, dim3((unsigned)nb), dim3(256), 0, s, y_perm, slot_pos, gates,
                               residual, shared, out, T, cpr, k, tpb, c0, w);
    }
}

}  // namespace moe
