// Route stage for gfx950: router logits, selection scores, top-k, gates and
// router probabilities.
//
// The router is an inner product per (token, expert) in fp32 (CS25
// "Lecture29" notes, section "Top-two routing": z = W_r x; CS336 lecture 4
// notes, section 5: the router is a single inner product, and section 11:
// computed in float32).  Because the selection is an integer decision taken on
// these fp32 values, every dot product walks its reduction index in order with
// one fma per step from +0 (no split-K, no MFMA whose internal summation order
// is unspecified), and the score transforms use the canonical functions of
// canon_math.h.  This file is compiled with -ffp-contract=off.
//
// Kernels
//   k_router_dots   SIMT register-blocked tile GEMM  x[T][d] . W[NC][d]^T -> dots[T][NC]
//                   (NC = E, or 2E for the noisy gate whose second half is x W_noise)
//   k_select        G lanes per token: scores (or hashed keys), k passes of a segmented arg-max,
//                   gates, router probabilities, per-block P partial sums
//   k_reduce_P      fixed-order two-level sum of the per-block partials -> P[E]
//   k_balance       (when requested) z-loss, importance and load partials;
//                   k_column_sums, k_seq_aux, k_balance_final reduce them
//   k_update_bias   the auxiliary-loss-free bias step
//   k_select_hier   hierarchical gate: groups, then experts inside each group
//   k_reroute       capacity reroute of the overflowing assignments (one block)
//   k_ec_scores, k_ec_select   expert choice: router probabilities, and each
//                   expert's top-C tokens by radix select
#include "device_common.h"
#include "canon_math.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// router dot products
// ---------------------------------------------------------------------------

// Tile: BT tokens x BE columns, K staged through LDS in chunks of KC
// (double buffered; the next chunk's global loads are in flight while the
// current chunk is consumed).  Thread (tg, cg) owns tokens tg + NTG*a and
// columns cg + NCG*b; for every output it walks i = 0..d-1 in order with one
// fma per step.  LDS rows are padded by 4 floats so the 16-byte reads of
// eight different rows fall in distinct banks.
template <int TT, int EE, int BE, int NT, int KC, bool BF16>
__global__ __launch_bounds__(NT) void k_router_dots(const void* __restrict__ x, const float* __restrict__ w0,
                                                    const float* __restrict__ w1, int T, int d, int E, int NC,
                                                    float* __restrict__ dots, int32_t* __restrict__ zero_word) {
    if (zero_word && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) zero_word[0] = 0;
    constexpr int LD = KC + 4;
    constexpr int NCG = BE / EE;          // column groups
    constexpr int NTG = NT / NCG;         // token groups
    constexpr int BT = NTG * TT;
    constexpr int XV = BF16 ? 8 : 4;      // x elements per 16-byte load
    constexpr int XCH = BT * KC / XV;     // 16-byte x chunks per K chunk
    constexpr int WCH = BE * KC / 4;      // 16-byte w chunks per K chunk
    constexpr int XPT = (XCH + NT - 1) / NT, WPT = (WCH + NT - 1) / NT;
    __shared__ __align__(16) float xs[2][BT * LD];
    __shared__ __align__(16) float wsh[2][BE * LD];

    const int tid = threadIdx.x;
    const int cg = tid % NCG, tg = tid / NCG;
    const int t0 = blockIdx.x * BT;
    const int c0 = blockIdx.y * BE;

    u32x4_t rx[XPT], rw[WPT];
    auto load = [&](int k0) {
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int ch = tid + q * NT;
            if (ch < XCH) {
                const int r = ch / (KC / XV), i = (ch % (KC / XV)) * XV;
                const int t = min(t0 + r, T - 1);
                rx[q] = *(const u32x4_t*)((const uint8_t*)x + ((int64_t)t * d + k0 + i) * (BF16 ? 2 : 4));
            }
        }
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int ch = tid + q * NT;
            if (ch < WCH) {
                const int r = ch / (KC / 4), i = (ch % (KC / 4)) * 4;
                const int c = min(c0 + r, NC - 1);
                const float* wr = c < E ? w0 + (int64_t)c * d : w1 + (int64_t)(c - E) * d;
                rw[q] = *(const u32x4_t*)(wr + k0 + i);
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int ch = tid + q * NT;
            if (ch < XCH) {
                const int r = ch / (KC / XV), i = (ch % (KC / XV)) * XV;
                float* dst = &xs[buf][r * LD + i];
                if constexpr (BF16) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        dst[2 * h] = bf16_bits_to_f32(rx[q][h] & 0xffffu);
                        dst[2 * h + 1] = bf16_bits_to_f32(rx[q][h] >> 16);
                    }
                } else {
                    *(u32x4_t*)dst = rx[q];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int ch = tid + q * NT;
            if (ch < WCH) {
                const int r = ch / (KC / 4), i = (ch % (KC / 4)) * 4;
                *(u32x4_t*)&wsh[buf][r * LD + i] = rw[q];
            }
        }
    };

    float acc[TT][EE];
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < EE; ++b) acc[a][b] = 0.0f;

    const int nch = d / KC;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        if (c + 1 < nch) load((c + 1) * KC);
#pragma unroll 4
        for (int i = 0; i < KC; i += 4) {
            float4 xv[TT], wv[EE];
#pragma unroll
            for (int a = 0; a < TT; ++a) xv[a] = *(const float4*)&xs[buf][(tg + NTG * a) * LD + i];
#pragma unroll
            for (int b = 0; b < EE; ++b) wv[b] = *(const float4*)&wsh[buf][(cg + NCG * b) * LD + i];
#pragma unroll
            for (int a = 0; a < TT; ++a)
#pragma unroll
                for (int b = 0; b < EE; ++b) {
                    float sacc = acc[a][b];
                    sacc = __builtin_fmaf(xv[a].x, wv[b].x, sacc);
                    sacc = __builtin_fmaf(xv[a].y, wv[b].y, sacc);
                    sacc = __builtin_fmaf(xv[a].z, wv[b].z, sacc);
                    sacc = __builtin_fmaf(xv[a].w, wv[b].w, sacc);
                    acc[a][b] = sacc;
                }
        }
        if (c + 1 < nch) store(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < TT; ++a) {
        const int t = t0 + tg + NTG * a;
        if (t >= T) continue;
#pragma unroll
        for (int b = 0; b < EE; ++b) {
            const int c = c0 + cg + NCG * b;
            if (c < NC) dots[(int64_t)t * NC + c] = acc[a][b];
        }
    }
}

// Few score columns (NC < 64), d a multiple of 128: one wave per block, one
// output per lane (BE columns x 64/BE tokens).  There are only T*NC/64 waves,
// at most a couple per CU, so nothing else runs while a wave waits for
// memory: K chunks of 128 are fetched S chunks ahead straight into a ring of
// LDS slots (direct-to-LDS loads, no staging registers, waits with fixed
// counts), and every output still walks i = 0..d-1 in order with one fma per
// step.  The rows of a slot are XOR swizzled in 16-byte chunks so that the
// lanes reading different rows at one k hit distinct banks.  Each slot is an
// LDS array of its own and the chunk loop is unrolled over the slots: with
// one array the compiler, unable to tell which bytes the loads in flight
// write, waited for all of them before some of the reads; this way most of
// its waits coincide with the fixed-count ones (it still drains part of the
// ring at a few slots).
template <int BE, bool BF16>
struct RingDots {
    static constexpr int KC = 128, BT = 64 / BE, XS = BF16 ? 2 : 4;
    static constexpr int XROW = KC * XS, WROW = KC * 4;      // bytes per row of a slot
    static constexpr int XB = BT * XROW, WB = BE * WROW;     // x and w bytes per slot
    static constexpr int XI = XB / 1024, WI = WB / 1024, NI = XI + WI;   // 1 KB loads per chunk
    static constexpr int SB = XB + WB;
    static constexpr int S_VM = 63 / NI + 1;                 // slots the vmcnt range allows
    static constexpr int S_LDS = 64 * 1024 / SB;             // slots within 64 KB of LDS
    static constexpr int S = S_VM < S_LDS ? (S_VM < 8 ? S_VM : 8) : (S_LDS < 8 ? S_LDS : 8);
    static constexpr bool ok = XB % 1024 == 0 && WB % 1024 == 0 && S >= 2;
};

template <int N>
__device__ __forceinline__ void dots_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <int BE, bool BF16>
__global__ __launch_bounds__(64) void k_router_dots_ring(const void* __restrict__ x, const float* __restrict__ w0,
                                                         const float* __restrict__ w1, int T, int d, int E, int NC,
                                                         float* __restrict__ dots, int32_t* __restrict__ zero_word) {
#if defined(__HIP_DEVICE_COMPILE__)
    (void)w1;
    if (zero_word && blockIdx.x == 0 && threadIdx.x == 0) zero_word[0] = 0;
    typedef RingDots<BE, BF16> P;
    constexpr int KC = P::KC, BT = P::BT, XS = P::XS, XROW = P::XROW, WROW = P::WROW, XB = P::XB;
    constexpr int XI = P::XI, WI = P::WI, NI = P::NI, SB = P::SB, S = P::S;
    constexpr int XCH = XROW / 16, WCH = WROW / 16;          // 16-byte chunks per row
    static_assert(P::ok, "shape does not tile into whole 1 KB loads");
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    static_assert(S <= 8, "at most 8 slots");
    __shared__ __align__(16) uint8_t sl0[SB], sl1[SB], sl2[SB], sl3[SB], sl4[SB], sl5[SB], sl6[SB], sl7[SB];
    auto slot = [&](int j) -> uint8_t* {
        return j == 0 ? sl0 : j == 1 ? sl1 : j == 2 ? sl2 : j == 3 ? sl3 : j == 4 ? sl4 : j == 5 ? sl5 : j == 6 ? sl6 : sl7;
    };

    const int lane = threadIdx.x;
    const int cg = lane % BE, tg = lane / BE;
    const int t0 = blockIdx.x * BT;
    const int nch = d / KC;

    // per-lane byte offset of each 1 KB load: x rows (tokens clamped to
    // T - 1), then w rows (columns clamped to NC - 1, NC == E here); LDS
    // chunk p of row r holds logical chunk p ^ (r mod chunks per row).
    // Buffer descriptors hold the bases, the chunk's K offset goes in the
    // scalar offset.
    constexpr int kRsrcWord3 = 0x00020000;
    const __amdgpu_buffer_rsrc_t rsx =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * d * XS), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsw =
        __builtin_amdgcn_make_buffer_rsrc((void*)w0, (short)0, (int)((int64_t)E * d * 4), kRsrcWord3);
    uint32_t offx[XI], offw[WI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int o = q * 1024 + 16 * lane;
        const int r = o / XROW, pc = (o % XROW) / 16;
        offx[q] = (uint32_t)(min(t0 + r, T - 1) * d * XS + ((pc ^ (r % XCH)) * 16));
    }
#pragma unroll
    for (int q = 0; q < WI; ++q) {
        const int o = q * 1024 + 16 * lane;
        const int r = o / WROW, pc = (o % WROW) / 16;
        offw[q] = (uint32_t)(min(r, NC - 1) * d * 4 + ((pc ^ (r % WCH)) * 16));
    }
    // chunk v goes to slot j = v % S (j is a compile-time constant at every
    // call); past the last chunk the last one is fetched again, so every
    // iteration issues NI loads
    auto issue = [&](int j, int v) {
        uint8_t* sl = slot(j);
        const int kc = min(v, nch - 1) * KC;
#pragma unroll
        for (int q = 0; q < XI; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_ptr_t)(sl + q * 1024), 16, offx[q], kc * XS, 0, 0);
#pragma unroll
        for (int q = 0; q < WI; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(sl + XB + q * 1024), 16, offw[q], kc * 4, 0, 0);
    };

#pragma unroll
    for (int v = 0; v < S - 1; ++v) issue(v, v);
    float acc = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += S) {
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const int c = c0 + j;
        // the slot of chunk c - 1 is rewritten below: its reads are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue((j + S - 1) % S, c + S - 1);
        dots_wait_vmcnt<(S - 1) * NI>();     // chunk c has landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (c >= nch) continue;              // past the end: loads only (uniform), no exit from the body
        const uint8_t* xrow = slot(j) + tg * XROW;
        const uint8_t* wrow = slot(j) + XB + cg * WROW;
        // 16-byte chunk q of this lane's x and w rows
        auto X = [&](int q) { return *(const u32x4_t*)(xrow + ((q ^ (tg % XCH)) * 16)); };
        auto W = [&](int q) { return *(const float4*)(wrow + ((q ^ (cg % WCH)) * 16)); };
        // the operands of 8 steps (k = 8g .. 8g + 7) are read PD groups
        // ahead into a ring of register sets, so a read's latency is covered
        // by the dependent fmas of the groups before (scheduling fences keep
        // the compiler from sinking the reads to their use)
        constexpr int NG = KC / 8, PD = 2;
        u32x4_t xf[PD + 1][BF16 ? 1 : 2];
        float4 wf[PD + 1][2];
        auto fetch = [&](int g, int b) {
            if constexpr (BF16) {
                xf[b][0] = X(g);
            } else {
                xf[b][0] = X(2 * g);
                xf[b][1] = X(2 * g + 1);
            }
            wf[b][0] = W(2 * g);
            wf[b][1] = W(2 * g + 1);
        };
#pragma unroll
        for (int g = 0; g < PD; ++g) fetch(g, g);
#pragma unroll
        for (int g = 0; g < NG; ++g) {          // 8 steps: k = 8g .. 8g + 7
            const int b = g % (PD + 1);
            if (g + PD < NG) fetch(g + PD, (g + PD) % (PD + 1));
            __builtin_amdgcn_sched_barrier(0);      // the reads stay ahead of this group's fmas
            const float4 wa = wf[b][0], wb = wf[b][1];
            float xv[8];
            if constexpr (BF16) {
                const u32x4_t v = xf[b][0];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xv[2 * h] = __uint_as_float(v[h] << 16);
                    xv[2 * h + 1] = __uint_as_float(v[h] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xv[h] = __uint_as_float(xf[b][0][h]);
                    xv[4 + h] = __uint_as_float(xf[b][1][h]);
                }
            }
            acc = __builtin_fmaf(xv[0], wa.x, acc);
            acc = __builtin_fmaf(xv[1], wa.y, acc);
            acc = __builtin_fmaf(xv[2], wa.z, acc);
            acc = __builtin_fmaf(xv[3], wa.w, acc);
            acc = __builtin_fmaf(xv[4], wb.x, acc);
            acc = __builtin_fmaf(xv[5], wb.y, acc);
            acc = __builtin_fmaf(xv[6], wb.z, acc);
            acc = __builtin_fmaf(xv[7], wb.w, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    dots_wait_vmcnt<0>();   // refetches of the last chunk may still be landing
    const int t = t0 + tg;
    if (t < T && cg < NC) dots[(int64_t)t * NC + cg] = acc;
#endif
}

// ---------------------------------------------------------------------------
// selection, gates, probabilities
// ---------------------------------------------------------------------------

// Pack (score order key, expert) so that a plain unsigned max picks the
// larger score and, on equal scores, the lower expert index.  0 is below
// every real candidate (a NaN score still packs above 0).
__device__ __forceinline__ uint64_t pack_cand(float key, int e) {
    const uint32_t ok = (uint32_t)canon::order_key(key) ^ 0x80000000u;
    return ((uint64_t)ok << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

template <int G>
__device__ __forceinline__ uint64_t seg_max_u64(uint64_t v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

template <int G>
__device__ __forceinline__ float seg_max_f(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

template <int G>
__device__ __forceinline__ float seg_sum_f(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
    return v;
}

// One pass of 256 threads handles 4 * (64 / G) tokens: lane = seg * G + g
// covers token seg of its wave and experts g, g + G, ..., g + G (V-1).
template <int G, int V>
__global__ __launch_bounds__(256) void k_select(const float* __restrict__ dots, int NC, const float* __restrict__ logit_bias,
                                                const float* __restrict__ sel_bias, const float* __restrict__ noise,
                                                const int32_t* __restrict__ token_ids, int gate, int T, int E, int k,
                                                uint64_t seed, uint64_t noise_offset, int32_t* __restrict__ topk_idx,
                                                float* __restrict__ topk_gate, float* __restrict__ scores,
                                                float* __restrict__ P_part, int32_t* __restrict__ status) {
    constexpr int SEGS = 64 / G;
    constexpr int TB = 4 * SEGS;
    __shared__ float red[4][V * G];

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int seg = lane / G, g = lane % G;
    const int t = blockIdx.x * TB + wave * SEGS + seg;
    const bool tok_ok = t < T;
    const bool hashed = gate == MOE_GATE_HASH;
    const uint32_t uid = (hashed && tok_ok) ? (uint32_t)token_ids[t] : 0u;

    float key[V], src[V], sig[V];
    bool valid[V];
    uint32_t taken = 0;
    int bad = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int e = g + G * v;
        valid[v] = tok_ok && e < E;
        key[v] = 0.0f; src[v] = 0.0f; sig[v] = 0.0f;
        if (!valid[v]) continue;
        if (hashed) {          // no router: the key is a hash of (token id, expert)
            key[v] = canon::hash_keyc(seed, noise_offset, (uint64_t)uid * (uint64_t)E + (uint64_t)e);
            if (scores) scores[(int64_t)t * E + e] = key[v];
            continue;
        }
        float z = dots[(int64_t)t * NC + e];
        if (logit_bias) z = z + logit_bias[e];
        float kv = z, sv = z;
        if (gate == MOE_GATE_NOISY_TOPK) {
            const float zn = dots[(int64_t)t * NC + E + e];
            const uint64_t flat = (uint64_t)t * (uint64_t)E + (uint64_t)e;
            const float n = noise ? noise[flat] : canon::normalc(seed, noise_offset, flat);
            kv = __builtin_fmaf(n, canon::softplusc(zn), z);
            sv = kv;
        } else if (gate == MOE_GATE_SIGMOID_BIAS) {
            const float s = canon::sigmoidc(z);
            sig[v] = s;
            kv = sel_bias ? s + sel_bias[e] : s;
        }
        key[v] = kv;
        src[v] = sv;
        if (!__builtin_isfinite(kv)) bad = 1;
        if (scores) scores[(int64_t)t * E + e] = kv;
    }

    // top-k: k passes of a segmented arg-max over the experts not yet taken
    // (loops run to the compile-time bound 16 so every array index is static)
    float src_sel[16], sig_sel[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        src_sel[j] = 0.0f; sig_sel[j] = 0.0f;
        if (j >= k) continue;
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (valid[v] && !((taken >> v) & 1u)) {
                const uint64_t c = pack_cand(key[v], g + G * v);
                best = c > best ? c : best;
            }
        best = seg_max_u64<G>(best);
        const int ew = (int)(0xffffffffu - (uint32_t)best);
        const int owner_g = ew % G, vw = ew / G;
        float s_own = 0.0f, sg_own = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (v == vw && g == owner_g) { s_own = src[v]; sg_own = sig[v]; taken |= 1u << v; }
        src_sel[j] = __shfl(s_own, seg * G + owner_g, 64);
        sig_sel[j] = __shfl(sg_own, seg * G + owner_g, 64);
        if (tok_ok && g == 0) topk_idx[(int64_t)t * k + j] = ew;
    }

    // softmax statistics over every expert (probabilities, full-softmax gate)
    float m_all = -__builtin_inff(), s_all = 0.0f;
    if (gate == MOE_GATE_SIGMOID_BIAS) {
#pragma unroll
        for (int v = 0; v < V; ++v) if (valid[v]) s_all = s_all + sig[v];
        s_all = seg_sum_f<G>(s_all);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) if (valid[v]) m_all = fmaxf(m_all, src[v]);
        m_all = seg_max_f<G>(m_all);
#pragma unroll
        for (int v = 0; v < V; ++v) if (valid[v]) s_all = s_all + canon::expc(src[v] - m_all);
        s_all = seg_sum_f<G>(s_all);
    }

    // gates
    if (tok_ok && g == 0) {
        float gv[16];
        if (hashed) {          // the selected experts' outputs are added
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = 1.0f;
        } else if (gate == MOE_GATE_SOFTMAX_FULL) {
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = canon::expc(src_sel[j] - m_all) / s_all;
        } else if (gate == MOE_GATE_SIGMOID_BIAS) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) if (j < k) s = s + sig_sel[j];
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = sig_sel[j] / s;
        } else {
            const float m = src_sel[0];
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                gv[j] = canon::expc(src_sel[j] - m);
                if (j < k) s = s + gv[j];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = gv[j] / s;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j < k) topk_gate[(int64_t)t * k + j] = gv[j];
    }

    // router probabilities -> per-block partial sums of P, in a fixed order
    float pacc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        float p = 0.0f;
        if (valid[v]) {
            if (hashed) p = ((taken >> v) & 1u) ? 1.0f / (float)k : 0.0f;
            else p = gate == MOE_GATE_SIGMOID_BIAS ? sig[v] / s_all : canon::expc(src[v] - m_all) / s_all;
        }
        pacc[v] = p;
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int off = G; off < 64; off <<= 1) pacc[v] = pacc[v] + __shfl_xor(pacc[v], off, 64);
    if (seg == 0) {
#pragma unroll
        for (int v = 0; v < V; ++v) red[wave][g + G * v] = pacc[v];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const float s = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
        P_part[(int64_t)blockIdx.x * E + e] = s;
    }
    if (bad) status[0] = MOE_DEV_NONFINITE;  // benign race: every writer stores the same value
}

// out[e] = scale * (sum over b of part[b][e]) for the 64 experts of this
// block, with 16 waves: wave w sums its contiguous range of b with 8
// interleaved accumulators (8 loads in flight), then the 8 and the 16 wave
// sums are added in a fixed order, so the result does not depend on timing.
__device__ __forceinline__ void column_sums(const float* __restrict__ part, int nblocks, int E, float scale,
                                            float* __restrict__ out_ws, float* __restrict__ out_user) {
    __shared__ float sums[16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int chunk = (nblocks + 15) / 16;
    const int b0 = min(nblocks, w * chunk), b1 = min(nblocks, b0 + chunk);
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f, a4 = 0.0f, a5 = 0.0f, a6 = 0.0f, a7 = 0.0f, r = 0.0f;
    if (e < E) {
        const float* src = part + e;
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
            a0 = a0 + src[(int64_t)(b + 0) * E];
            a1 = a1 + src[(int64_t)(b + 1) * E];
            a2 = a2 + src[(int64_t)(b + 2) * E];
            a3 = a3 + src[(int64_t)(b + 3) * E];
            a4 = a4 + src[(int64_t)(b + 4) * E];
            a5 = a5 + src[(int64_t)(b + 5) * E];
            a6 = a6 + src[(int64_t)(b + 6) * E];
            a7 = a7 + src[(int64_t)(b + 7) * E];
        }
        for (; b < b1; ++b) r = r + src[(int64_t)b * E];
    }
    sums[w][lane] = (((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7))) + r;
    __syncthreads();
    if (w == 0 && e < E) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) t = t + sums[i][lane];
        t = t * scale;
        if (out_ws) out_ws[e] = t;
        if (out_user) out_user[e] = t;
    }
}

// P[e] = (sum of the per-block partials) / T, and the device status copy.
__global__ __launch_bounds__(1024) void k_reduce_P(const float* __restrict__ P_part, int nblocks, int E, int T,
                                                   float* __restrict__ P_ws, float* __restrict__ P_out,
                                                   const int32_t* __restrict__ status_ws,
                                                   int32_t* __restrict__ status_out) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && status_out) status_out[0] = status_ws[0];
    column_sums(P_part, nblocks, E, T > 0 ? 1.0f / (float)T : 0.0f, P_ws, P_out);
}

// Plain column sums (importance, load, z-loss partials).
__global__ __launch_bounds__(1024) void k_column_sums(const float* __restrict__ part, int nblocks, int E, float scale,
                                                      float* __restrict__ out_ws, float* __restrict__ out_user) {
    column_sums(part, nblocks, E, scale, out_ws, out_user);
}

// Hierarchical gate (two levels): one wave per token, 4 tokens per block.
// Lanes hold the primary logits of the n_groups groups (columns E .. E+A-1
// of the router product); KP passes of a wave arg-max pick the groups (ties
// to the lower index), then for each picked group its B secondary logits
// (columns g B .. g B + B-1, plus the logit bias) give KS more passes.  Gates:
// softmax over the picked primary logits times softmax over the picked
// secondary logits of the group, in fp32 with the canonical exp.  Router
// probabilities softmax(zp)_g * softmax(z of group g)_j for every expert, summed
// per block in wave order.
__global__ __launch_bounds__(256) void k_select_hier(const float* __restrict__ dots, int NC,
                                                     const float* __restrict__ logit_bias, int T, int E, int A, int KP,
                                                     int KS, int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_gate, float* __restrict__ scores,
                                                     float* __restrict__ P_part, int32_t* __restrict__ status) {
    __shared__ float pw[4][1024];      // router probabilities per wave (token)
    __shared__ float gstat[4][64][2];  // per group: max and sum of exp of its secondary logits
    __shared__ float pprob[4][64];     // primary probabilities softmax(zp)
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const int B = E / A, k = KP * KS;
    const float ninf = -__builtin_inff();
    int bad = 0;
    if (t < T) {
        const float* zr = dots + (int64_t)t * NC;
        auto zsec = [&](int e) { return logit_bias ? zr[e] + logit_bias[e] : zr[e]; };
        for (int e = lane; e < E; e += 64) {
            const float z = zsec(e);
            if (!__builtin_isfinite(z)) bad = 1;
            if (scores) scores[(int64_t)t * E + e] = z;
        }
        const float zp = lane < A ? zr[E + lane] : ninf;
        if (lane < A && !__builtin_isfinite(zp)) bad = 1;
        // primary softmax over all groups (probabilities)
        const float mp = seg_max_f<64>(zp);
        const float sp = seg_sum_f<64>(lane < A ? canon::expc(zp - mp) : 0.0f);
        if (lane < A) pprob[wave][lane] = canon::expc(zp - mp) / sp;
        // per-group softmax statistics of the secondary logits
        for (int g = 0; g < A; ++g) {
            const float z = lane < B ? zsec(g * B + lane) : ninf;
            const float m = seg_max_f<64>(z);
            const float sm = seg_sum_f<64>(lane < B ? canon::expc(z - m) : 0.0f);
            if (lane == 0) { gstat[wave][g][0] = m; gstat[wave][g][1] = sm; }
        }
        // pick the groups
        bool taken = false;
        int grp[16];
        float zps[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            grp[j] = 0; zps[j] = 0.0f;
            if (j >= KP) continue;
            const uint64_t best = seg_max_u64<64>((lane < A && !taken) ? pack_cand(zp, lane) : 0ull);
            const int g = (int)(0xffffffffu - (uint32_t)best);
            grp[j] = g;
            zps[j] = __shfl(zp, g, 64);
            if (lane == g) taken = true;
        }
        float gp[16], sgp = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            gp[j] = canon::expc(zps[j] - zps[0]);
            if (j < KP) sgp = sgp + gp[j];
        }
        // pick the experts inside each picked group
        for (int j = 0; j < KP; ++j) {
            const int g = grp[j];
            const float z = lane < B ? zsec(g * B + lane) : ninf;
            bool tk = false;
            int ex[16];
            float zs[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                ex[q] = 0; zs[q] = 0.0f;
                if (q >= KS) continue;
                const uint64_t best = seg_max_u64<64>((lane < B && !tk) ? pack_cand(z, lane) : 0ull);
                const int jj = (int)(0xffffffffu - (uint32_t)best);
                ex[q] = g * B + jj;
                zs[q] = __shfl(z, jj, 64);
                if (lane == jj) tk = true;
            }
            float gs[16], sgs = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                gs[q] = canon::expc(zs[q] - zs[0]);
                if (q < KS) sgs = sgs + gs[q];
            }
            if (lane == 0) {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (q < KS) {
                        topk_idx[(int64_t)t * k + j * KS + q] = ex[q];
                        topk_gate[(int64_t)t * k + j * KS + q] = (gp[j] / sgp) * (gs[q] / sgs);
                    }
            }
        }
        for (int e = lane; e < E; e += 64) {
            const int g = e / B;
            pw[wave][e] = pprob[wave][g] * (canon::expc(zsec(e) - gstat[wave][g][0]) / gstat[wave][g][1]);
        }
    } else {
        for (int e = lane; e < E; e += 64) pw[wave][e] = 0.0f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        P_part[(int64_t)blockIdx.x * E + e] = ((pw[0][e] + pw[1][e]) + pw[2][e]) + pw[3][e];
    if (bad) status[0] = MOE_DEV_NONFINITE;   // benign race: every writer stores the same value
}

int hier_select_blocks(int T) { return (T + 3) / 4; }

void launch_select_hier(const float* dots, int NC, const float* logit_bias, int T, int E, int A, int KP, int KS,
                        int32_t* topk_idx, float* topk_gate, float* scores, float* P_part, int32_t* status,
                        hipStream_t s) {
    if (T <= 0) return;
    hipLaunchKernelGGL(k_select_hier, dim3(hier_select_blocks(T)), dim3(256), 0, s, dots, NC, logit_bias, T, E, A, KP,
                       KS, topk_idx, topk_gate, scores, P_part, status);
}

// Capacity reroute, one block.  The assignments past their expert's
// capacity (slot_pos < 0 after the capacity cut) are compacted chunk by
// chunk in (t, j) order.  All 16 waves then rank, for each of them, the
// experts its token does not hold: all of them when E <= 64 (lane e counts
// the keys above its own, read back from LDS), else the 16 best (wave
// arg-max passes), and copy
// the token's experts into LDS.  Wave 0 finally takes the entries one at a
// time in order: lane q tests ranked expert q, and the first one that still
// has room and is not held by then wins; when a truncated list is exhausted
// a scan of all the token's experts decides.  Only moves of the same token
// change what it holds, and its slots are consecutive, so the held set is
// carried in registers from one slot to the next (also across chunks); the
// next entry's lists are read ahead; moves are device-scope stores, waited
// for at the end of each chunk.
constexpr int kRerouteCand = 64;
constexpr int kRerouteChunk = 256;
constexpr int kRerouteWaves = 8;

__global__ __launch_bounds__(kRerouteWaves * 64) void k_reroute(int32_t* __restrict__ idx, const float* __restrict__ keys,
                                                  const int32_t* __restrict__ slot_pos,
                                                  const int32_t* __restrict__ offsets, int T, int E, int k,
                                                  int32_t C) {
    __shared__ int32_t room[1024];
    __shared__ int32_t list[kRerouteChunk];
    __shared__ int32_t cand[kRerouteChunk][kRerouteCand];
    __shared__ int32_t hold[kRerouteChunk][16];
    __shared__ int32_t trunc_[kRerouteChunk];
    __shared__ int32_t tokl[kRerouteChunk];      // token of each entry
    __shared__ int32_t wcount[kRerouteWaves];
    __shared__ uint64_t rk[kRerouteWaves][64];   // per wave: the 64 packed keys being ranked
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int e = tid; e < E; e += kRerouteWaves * 64) room[e] = C - (offsets[e + 1] - offsets[e]);
    __syncthreads();
    auto held = [&](const int32_t (&cur)[16], int e) {
        bool h = false;
#pragma unroll
        for (int j = 0; j < 16; ++j) h = h || cur[j] == e;
        return h;
    };
    int64_t t_prev = -1;
    int32_t cur[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) cur[j] = -1;
    const int64_t na = (int64_t)T * k;
    for (int64_t a0 = 0; a0 < na; a0 += kRerouteChunk) {
        // 1. ordered list of the chunk's overflowing assignments
        const int64_t a = a0 + tid;
        bool ov = false;
        if (tid < kRerouteChunk && a < na) {
            const int32_t e = idx[a];
            ov = slot_pos[a] < 0 && e >= 0 && e < E;
        }
        const uint64_t m = __ballot(ov);
        if (lane == 0) wcount[w] = __popcll(m);
        __syncthreads();
        int base = 0, tot = 0;
        for (int q = 0; q < kRerouteWaves; ++q) {
            if (q < w) base += wcount[q];
            tot += wcount[q];
        }
        if (ov) list[base + __popcll(m & ((1ull << lane) - 1ull))] = tid;
        __syncthreads();
        // 2. per entry: the token's experts, and the experts it does not hold, ranked
        for (int i = w; i < tot; i += kRerouteWaves) {
            const int t = (int)(a0 + list[i]) / k;     // T k < 2^31
            if (lane == 0) tokl[i] = t;
            int32_t ids[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                ids[j] = j < k ? __hip_atomic_load(&idx[(int64_t)t * k + j], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : -1;
            if (lane < 16) hold[i][lane] = ids[lane < 16 ? lane : 0];
            if (E <= 64) {
                const uint64_t mine = (lane < E && !held(ids, lane)) ? pack_cand(keys[(int64_t)t * E + lane], lane) : 0ull;
                rk[w][lane] = mine;
                int rank = 0;
#pragma unroll 16
                for (int j = 0; j < 64; ++j) rank += rk[w][j] > mine ? 1 : 0;   // broadcast LDS reads
                const int n_elig = __popcll(__ballot(mine != 0ull));
                if (lane >= n_elig) cand[i][lane] = -1;
                if (mine) cand[i][rank] = lane;
                if (lane == 0) trunc_[i] = 0;
            } else {
                uint64_t kc[16];    // (key, index) of experts lane + 64 v, 0 when held or absent
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int e = lane + 64 * v;
                    kc[v] = (e < E && !held(ids, e)) ? pack_cand(keys[(int64_t)t * E + e], e) : 0ull;
                }
                int last = -1;
                for (int q = 0; q < 16; ++q) {
                    uint64_t best = 0;
#pragma unroll
                    for (int v = 0; v < 16; ++v) best = kc[v] > best ? kc[v] : best;
                    best = seg_max_u64<64>(best);
                    const int e = best ? (int)(0xffffffffu - (uint32_t)best) : -1;
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (e >= 0 && e == lane + 64 * v) kc[v] = 0ull;
                    if (lane == 0) cand[i][q] = e;
                    last = e;
                }
                if (lane >= 16) cand[i][lane] = -1;
                if (lane == 0) trunc_[i] = last >= 0 ? 1 : 0;   // more experts may lie beyond the 16
            }
        }
        __syncthreads();
        // 3. the moves, in order
        if (w == 0 && tot > 0) {
            int32_t n_list = list[0], n_cand = cand[0][lane], n_trunc = trunc_[0], n_tok = tokl[0];
            for (int i = 0; i < tot; ++i) {
                const int64_t a1 = a0 + n_list;
                const int t = n_tok;
                const int32_t e_l = n_cand, tr = n_trunc;
                if (t != t_prev) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) cur[j] = hold[i][j];
                    t_prev = t;
                }
                if (i + 1 < tot) {          // read the next entry ahead
                    n_list = list[i + 1];
                    n_cand = cand[i + 1][lane];
                    n_trunc = trunc_[i + 1];
                    n_tok = tokl[i + 1];
                }
                const bool ok = e_l >= 0 && room[e_l] > 0 && !held(cur, e_l);
                const uint64_t okm = __ballot(ok);
                int chosen = -1;
                if (okm) {
                    chosen = __shfl(e_l, __ffsll((unsigned long long)okm) - 1, 64);
                } else if (tr) {
                    // every ranked expert is taken: scan all of them
                    uint64_t best = 0;
                    for (int e = lane; e < E; e += 64) {
                        if (room[e] <= 0 || held(cur, e)) continue;
                        const uint64_t c = pack_cand(keys[(int64_t)t * E + e], e);
                        best = c > best ? c : best;
                    }
                    best = seg_max_u64<64>(best);
                    if (best) chosen = (int)(0xffffffffu - (uint32_t)best);
                }
                if (chosen >= 0) {
                    if (lane == 0) {
                        __hip_atomic_store(&idx[a1], chosen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        room[chosen] -= 1;
                    }
                    const int js = (int)(a1 - (int64_t)t * k);
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (j == js) cur[j] = chosen;
                }
            }
            // the moves are visible before the next chunk reads token ids
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
    }
}

void launch_reroute(int32_t* idx, const float* keys, const int32_t* slot_pos, const int32_t* offsets, int T, int E,
                    int k, int64_t C, hipStream_t s) {
    if (T <= 0 || C < 0) return;
    hipLaunchKernelGGL(k_reroute, dim3(1), dim3(kRerouteWaves * 64), 0, s, idx, keys, slot_pos, offsets, T, E, k,
                       (int32_t)C);
}

// ---------------------------------------------------------------------------
// balance and stability statistics (after k_select, when requested)
// ---------------------------------------------------------------------------

// Standard normal CDF, Phi(x) = erfc(-x / sqrt 2) / 2.
__device__ __forceinline__ float phi_f(float x) { return 0.5f * erfcf(-x * 0.70710678118654752f); }

// Same lane mapping as k_select.  Per token: the squared log-sum-exp of the
// clean logits; every expert's received gate (importance) and, for the noisy
// gate, Phi((z_e - kth_excluding(H, k, e)) / softplus(zn_e)) (load).  The
// noisy scores H are recomputed with the same canonical functions and noise
// as in k_select, so they are bit-identical to the ones the selection used.
// kth_excluding is the (k+1)-th largest H for a selected expert and the k-th
// largest (the smallest selected one) otherwise.  Per-block partial sums in a
// fixed order.
template <int G, int V>
__global__ __launch_bounds__(256) void k_balance(const float* __restrict__ dots, int NC,
                                                 const float* __restrict__ logit_bias, const float* __restrict__ noise,
                                                 int gate, int T, int E, int k, uint64_t seed, uint64_t noise_offset,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ topk_gate, float* __restrict__ imp_part,
                                                 float* __restrict__ load_part, float* __restrict__ cnt_part,
                                                 float* __restrict__ z_part) {
    constexpr int SEGS = 64 / G;
    __shared__ float red_i[4][V * G];
    __shared__ float red_l[4][V * G];
    __shared__ float red_c[4][V * G];
    __shared__ float red_z[4];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int seg = lane / G, g = lane % G;
    const int t = blockIdx.x * (4 * SEGS) + wave * SEGS + seg;
    const bool tok_ok = t < T;
    const bool noisy = gate == MOE_GATE_NOISY_TOPK;

    float z[V], key[V], sc[V], imp[V];
    bool valid[V], sel[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int e = g + G * v;
        valid[v] = tok_ok && e < E;
        z[v] = 0.0f; key[v] = 0.0f; sc[v] = 1.0f; imp[v] = 0.0f; sel[v] = false;
        if (!valid[v]) continue;
        float zz = dots[(int64_t)t * NC + e];
        if (logit_bias) zz = zz + logit_bias[e];
        z[v] = zz;
        key[v] = zz;
        if (noisy) {
            const float zn = dots[(int64_t)t * NC + E + e];
            const uint64_t flat = (uint64_t)t * (uint64_t)E + (uint64_t)e;
            const float n = noise ? noise[flat] : canon::normalc(seed, noise_offset, flat);
            sc[v] = canon::softplusc(zn);
            key[v] = __builtin_fmaf(n, sc[v], zz);
        }
    }
    // selected experts and their gates
    if (tok_ok) {
        for (int j = 0; j < k; ++j) {
            const int ej = topk_idx[(int64_t)t * k + j];
            const float gj = topk_gate[(int64_t)t * k + j];
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (valid[v] && ej == g + G * v) { sel[v] = true; imp[v] = gj; }
        }
    }
    // log-sum-exp of the clean logits
    float m = -__builtin_inff(), sm = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) if (valid[v]) m = fmaxf(m, z[v]);
    m = seg_max_f<G>(m);
#pragma unroll
    for (int v = 0; v < V; ++v) if (valid[v]) sm = sm + canon::expc(z[v] - m);
    sm = seg_sum_f<G>(sm);
    const float lse = m + canon::logc(sm);
    float zterm = (tok_ok && g == 0) ? lse * lse : 0.0f;
    // smooth load (noisy gate)
    float ld[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ld[v] = 0.0f;
    if (noisy) {
        float kth = __builtin_inff(), nxt = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (valid[v]) {
                if (sel[v]) kth = fminf(kth, key[v]);
                else nxt = fmaxf(nxt, key[v]);
            }
        kth = -seg_max_f<G>(-kth);
        nxt = seg_max_f<G>(nxt);
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (valid[v]) ld[v] = k >= E ? 1.0f : phi_f((z[v] - (sel[v] ? nxt : kth)) / sc[v]);
    }
    // per-block partials, fixed order: across the segments of a wave, then the
    // 4 waves (selection counts are small integers, exact in fp32)
    float cn[V];
#pragma unroll
    for (int v = 0; v < V; ++v) cn[v] = sel[v] ? 1.0f : 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int off = G; off < 64; off <<= 1) {
            imp[v] = imp[v] + __shfl_xor(imp[v], off, 64);
            ld[v] = ld[v] + __shfl_xor(ld[v], off, 64);
            cn[v] = cn[v] + __shfl_xor(cn[v], off, 64);
        }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) zterm = zterm + __shfl_xor(zterm, off, 64);
    if (seg == 0) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            red_i[wave][g + G * v] = imp[v];
            red_l[wave][g + G * v] = ld[v];
            red_c[wave][g + G * v] = cn[v];
        }
    }
    if (lane == 0) red_z[wave] = zterm;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        imp_part[(int64_t)blockIdx.x * E + e] = ((red_i[0][e] + red_i[1][e]) + red_i[2][e]) + red_i[3][e];
        if (noisy) load_part[(int64_t)blockIdx.x * E + e] = ((red_l[0][e] + red_l[1][e]) + red_l[2][e]) + red_l[3][e];
        cnt_part[(int64_t)blockIdx.x * E + e] = ((red_c[0][e] + red_c[1][e]) + red_c[2][e]) + red_c[3][e];
    }
    if (threadIdx.x == 0) z_part[blockIdx.x] = ((red_z[0] + red_z[1]) + red_z[2]) + red_z[3];
}

// Fixed-tree sum of one value per thread over a block of 256 threads.
__device__ __forceinline__ float block_sum_256(float v, float* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int half = 128; half >= 1; half >>= 1) {
        if ((int)threadIdx.x < half) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + half];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

// Sequence s (tokens [s L, (s+1) L), blocks [s nb, (s+1) nb) of k_select /
// k_balance): E * sum_e f_e P_e with f_e = n_e / (L k) and P_e the mean
// router probability, both summed from the per-block partials with 8
// interleaved accumulators in a fixed order.  With whole_call the sequence
// is the whole call and the already reduced counts and mean P are used.
__device__ __forceinline__ float sum_blocks(const float* __restrict__ part, int b0, int b1, int E, int e) {
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f, a4 = 0.0f, a5 = 0.0f, a6 = 0.0f, a7 = 0.0f, r = 0.0f;
    const float* src = part + e;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
        a0 = a0 + src[(int64_t)(b + 0) * E];
        a1 = a1 + src[(int64_t)(b + 1) * E];
        a2 = a2 + src[(int64_t)(b + 2) * E];
        a3 = a3 + src[(int64_t)(b + 3) * E];
        a4 = a4 + src[(int64_t)(b + 4) * E];
        a5 = a5 + src[(int64_t)(b + 5) * E];
        a6 = a6 + src[(int64_t)(b + 6) * E];
        a7 = a7 + src[(int64_t)(b + 7) * E];
    }
    for (; b < b1; ++b) r = r + src[(int64_t)b * E];
    return (((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7))) + r;
}

__global__ __launch_bounds__(256) void k_seq_aux(const float* __restrict__ cnt_part, const float* __restrict__ P_part,
                                                 const float* __restrict__ cnt_all, const float* __restrict__ P_mean,
                                                 int L, int k, int E, int nb_cnt, int nb_p,
                                                 float* __restrict__ seq_part) {
    __shared__ float red[256];
    const int s = blockIdx.x;
    float acc = 0.0f;
    for (int e = threadIdx.x; e < E; e += 256) {
        const float n = cnt_all ? cnt_all[e] : sum_blocks(cnt_part, s * nb_cnt, (s + 1) * nb_cnt, E, e);
        const float pm = P_mean ? P_mean[e] : sum_blocks(P_part, s * nb_p, (s + 1) * nb_p, E, e) / (float)L;
        acc = acc + (n / (float)(L * k)) * pm;
    }
    const float tot = block_sum_256(acc, red);
    if (threadIdx.x == 0) seq_part[s] = (float)E * tot;
}

// Scalars: CV^2 of importance and load (population variance / mean^2), the
// z-loss and the mean of the per-sequence balance terms.
__global__ __launch_bounds__(256) void k_balance_final(const float* __restrict__ imp, const float* __restrict__ load,
                                                       const float* __restrict__ z_total, const float* __restrict__ seq_part,
                                                       int nseq, int E, float* __restrict__ imp_cv2,
                                                       float* __restrict__ load_cv2, float* __restrict__ z_loss,
                                                       float* __restrict__ seq_aux) {
    __shared__ float red[256];
    for (int pass = 0; pass < 2; ++pass) {
        const float* v = pass == 0 ? imp : load;
        float* out = pass == 0 ? imp_cv2 : load_cv2;
        if (!v) continue;
        float s = 0.0f;
        for (int e = threadIdx.x; e < E; e += 256) s = s + v[e];
        const float mean = block_sum_256(s, red) / (float)E;
        float q = 0.0f;
        for (int e = threadIdx.x; e < E; e += 256) q = q + (v[e] - mean) * (v[e] - mean);
        const float var = block_sum_256(q, red) / (float)E;
        if (threadIdx.x == 0 && out) out[0] = mean != 0.0f ? var / (mean * mean) : 0.0f;
    }
    float a = 0.0f;
    for (int i = threadIdx.x; i < nseq; i += 256) a = a + seq_part[i];
    const float tot = block_sum_256(a, red);
    if (threadIdx.x == 0) {
        if (z_loss) z_loss[0] = z_total[0];
        if (seq_aux) seq_aux[0] = nseq > 0 ? tot / (float)nseq : 0.0f;
    }
}

// b_e += gamma * sign(mean - n_e), the comparison n_e * E <=> sum n exact in
// integers.
__global__ __launch_bounds__(1024) void k_update_bias(const int32_t* __restrict__ counts, int E, float gamma,
                                                      float* __restrict__ bias) {
    __shared__ int64_t red[1024];
    int64_t s = 0;
    for (int e = threadIdx.x; e < E; e += 1024) s += counts[e];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int half = 512; half >= 1; half >>= 1) {
        if ((int)threadIdx.x < half) red[threadIdx.x] += red[threadIdx.x + half];
        __syncthreads();
    }
    const int64_t total = red[0];
    for (int e = threadIdx.x; e < E; e += 1024) {
        const int64_t c = (int64_t)counts[e] * E;
        if (c < total) bias[e] = bias[e] + gamma;
        else if (c > total) bias[e] = bias[e] - gamma;
    }
}

__global__ void k_copy_status(const int32_t* __restrict__ status_ws, int32_t* __restrict__ status_out) {
    if (threadIdx.x == 0 && status_out) status_out[0] = status_ws[0];
}

__global__ void k_zero_i32(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// expert choice
// ---------------------------------------------------------------------------

// S[t][e] = softmax over the experts of z[t] (+ logit bias): one thread per
// token, m = max, s = sum over e = 0..E-1 in order of exp(z_e - m) with the
// canonical exp, S_e = exp(z_e - m) / s (correctly rounded fp32 division), so
// the scores, and hence the selection, are reproducible bit for bit.
__global__ __launch_bounds__(256) void k_ec_scores(const float* __restrict__ dots, const float* __restrict__ logit_bias,
                                                   int T, int E, float* __restrict__ S,
                                                   int32_t* __restrict__ status) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const float* z = dots + (int64_t)t * E;
    float m = -__builtin_inff();
    for (int e = 0; e < E; ++e) m = fmaxf(m, logit_bias ? z[e] + logit_bias[e] : z[e]);
    float s = 0.0f;
    for (int e = 0; e < E; ++e) s = s + canon::expc((logit_bias ? z[e] + logit_bias[e] : z[e]) - m);
    int bad = 0;
    for (int e = 0; e < E; ++e) {
        const float v = canon::expc((logit_bias ? z[e] + logit_bias[e] : z[e]) - m) / s;
        if (!__builtin_isfinite(v)) bad = 1;
        S[(int64_t)t * E + e] = v;
    }
    if (bad) status[0] = MOE_DEV_NONFINITE;   // benign race: every writer stores the same value
}

// Expert e (one block of 1024 threads) takes the C tokens with the largest
// S[., e], ties to the lower token index.  S >= 0, so its bit pattern orders
// like the value: a 4-pass radix select (8 bits per pass, most significant
// first) finds the C-th largest key K; every token above K is taken, and the
// first `need` tokens equal to K in index order (an exclusive scan over the
// tokens in chunks of 1024).  Integer histograms: the result does not depend
// on timing.
__global__ __launch_bounds__(1024) void k_ec_select(const float* __restrict__ S, int T, int E, int C,
                                                    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
    __shared__ int32_t hist[256];
    __shared__ int32_t sel_digit, sel_above;
    __shared__ int32_t scan[1024];
    const int e = blockIdx.x, tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int need = C;                                  // tokens still to take at or below the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += 1024) hist[i] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += 1024) {
            const uint32_t u = __float_as_uint(S[(int64_t)t * E + e]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid == 0) {
            int above = 0, d = 255;
            for (; d > 0; --d) {
                if (above + hist[d] >= need) break;
                above += hist[d];
            }
            sel_digit = d;
            sel_above = above;
        }
        __syncthreads();
        prefix |= (uint32_t)sel_digit << shift;
        mask |= 255u << shift;
        need -= sel_above;
        __syncthreads();
    }
    // prefix is now the C-th largest key; take everything above it and the
    // first `need` tokens equal to it
    int carry = 0;
    for (int t0 = 0; t0 < T; t0 += 1024) {
        const int t = t0 + tid;
        uint32_t u = 0;
        float v = 0.0f;
        if (t < T) { v = S[(int64_t)t * E + e]; u = __float_as_uint(v); }
        const int eq = (t < T && u == prefix) ? 1 : 0;
        scan[tid] = eq;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int rank_eq = carry + scan[tid] - eq;   // equal tokens before t
        const int total_eq = scan[1023];
        if (t < T) {
            const bool take = u > prefix || (eq && rank_eq < need);
            topk_idx[(int64_t)t * E + e] = take ? e : -1;
            topk_gate[(int64_t)t * E + e] = take ? v : 0.0f;
        }
        carry += total_eq;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

static int pow2_at_least(int v) { int p = 1; while (p < v) p <<= 1; return p; }

template <bool BF16>
static void launch_dots_t(const void* x, const float* w0, const float* w1, int T, int d, int E, int NC, float* dots,
                          int32_t* zero_word, hipStream_t s) {
    if (NC > 32) {
        // (also 33 .. 63 columns: the few-column kernels below stop at 32)
        // 16 x TT tokens x 64 columns per block of 256 threads; TT is the
        // largest of 4, 2, 1 that still gives at least 512 blocks (two per CU),
        // so that a CU has a second block to run while one waits on memory
        const int cb = (NC + 63) / 64;
        int TT = 4;
        while (TT > 1 && (int64_t)((T + 16 * TT - 1) / (16 * TT)) * cb < 512) TT /= 2;
        dim3 grid((T + 16 * TT - 1) / (16 * TT), cb);
        if (TT == 4)
            hipLaunchKernelGGL((k_router_dots<4, 4, 64, 256, 64, BF16>), grid, dim3(256), 0, s, x, w0, w1, T, d, E, NC,
                               dots, zero_word);
        else if (TT == 2)
            hipLaunchKernelGGL((k_router_dots<2, 4, 64, 256, 64, BF16>), grid, dim3(256), 0, s, x, w0, w1, T, d, E, NC,
                               dots, zero_word);
        else
            hipLaunchKernelGGL((k_router_dots<1, 4, 64, 256, 64, BF16>), grid, dim3(256), 0, s, x, w0, w1, T, d, E, NC,
                               dots, zero_word);
        return;
    }
    const int BE = pow2_at_least(NC);
    if (d % 128 == 0 && BE >= 2 && BE <= 16 && NC == E && (int64_t)T * d * (BF16 ? 2 : 4) < (1ll << 31)) {
        dim3 grid((T + 64 / BE - 1) / (64 / BE), 1);
        switch (BE) {
            case 2: hipLaunchKernelGGL((k_router_dots_ring<2, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E, NC, dots, zero_word); break;
            case 4: hipLaunchKernelGGL((k_router_dots_ring<4, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E, NC, dots, zero_word); break;
            case 8: hipLaunchKernelGGL((k_router_dots_ring<8, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E, NC, dots, zero_word); break;
            default: hipLaunchKernelGGL((k_router_dots_ring<16, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E, NC, dots, zero_word); break;
        }
        return;
    }
    const int BT = 64 / BE;
    dim3 grid((T + BT - 1) / BT, 1);
    // K chunks of 128 when d allows it, else 64 (d is a multiple of 64)
    const bool k128 = d % 128 == 0;
    switch (BE) {
#define MOE_DOTS_CASE(B)                                                                                        \
    case B:                                                                                                     \
        if (k128)                                                                                               \
            hipLaunchKernelGGL((k_router_dots<1, 1, B, 64, 128, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E, \
                               NC, dots, zero_word);                                                                     \
        else                                                                                                    \
            hipLaunchKernelGGL((k_router_dots<1, 1, B, 64, 64, BF16>), grid, dim3(64), 0, s, x, w0, w1, T, d, E,  \
                               NC, dots, zero_word);                                                                     \
        break;
        MOE_DOTS_CASE(1) MOE_DOTS_CASE(2) MOE_DOTS_CASE(4) MOE_DOTS_CASE(8) MOE_DOTS_CASE(16) MOE_DOTS_CASE(32)
#undef MOE_DOTS_CASE
    }
}

void launch_router_dots(bool bf16, const void* x, const float* w0, const float* w1, int T, int d, int E, int NC,
                        float* dots, hipStream_t s, int32_t* zero_word) {
    if (T <= 0) {
        if (zero_word) launch_zero_i32(zero_word, 1, s);
        return;
    }
    if (bf16) launch_dots_t<true>(x, w0, w1, T, d, E, NC, dots, zero_word, s);
    else launch_dots_t<false>(x, w0, w1, T, d, E, NC, dots, zero_word, s);
}

int select_blocks(int T, int E) {
    const int G = E >= 64 ? 64 : pow2_at_least(E);
    const int TB = 4 * (64 / G);
    return (T + TB - 1) / TB;
}

void launch_select(const float* dots, int NC, const float* logit_bias, const float* sel_bias, const float* noise,
                   const int32_t* token_ids, int gate, int T, int E, int k, uint64_t seed, uint64_t noise_offset,
                   int32_t* topk_idx, float* topk_gate, float* scores, float* P_part, int32_t* status,
                   hipStream_t s) {
    if (T <= 0) return;
    const int G = E >= 64 ? 64 : pow2_at_least(E);
    const int V = (E + G - 1) / G;
    const int nb = select_blocks(T, E);
#define MOE_SEL_ARGS dots, NC, logit_bias, sel_bias, noise, token_ids, gate, T, E, k, seed, noise_offset, topk_idx, topk_gate, scores, P_part, status
#define MOE_SEL(GG, VV) hipLaunchKernelGGL((k_select<GG, VV>), dim3(nb), dim3(256), 0, s, MOE_SEL_ARGS)
    if (G < 64) {
        switch (G) {
            case 1: MOE_SEL(1, 1); break;
            case 2: MOE_SEL(2, 1); break;
            case 4: MOE_SEL(4, 1); break;
            case 8: MOE_SEL(8, 1); break;
            case 16: MOE_SEL(16, 1); break;
            default: MOE_SEL(32, 1); break;
        }
    } else if (V <= 1) MOE_SEL(64, 1);
    else if (V <= 2) MOE_SEL(64, 2);
    else if (V <= 4) MOE_SEL(64, 4);
    else if (V <= 8) MOE_SEL(64, 8);
    else MOE_SEL(64, 16);
#undef MOE_SEL
#undef MOE_SEL_ARGS
}

void launch_reduce_P(const float* P_part, int nblocks, int E, int T, float* P_ws, float* P_out,
                     const int32_t* status_ws, int32_t* status_out, hipStream_t s) {
    hipLaunchKernelGGL(k_reduce_P, dim3((E + 63) / 64), dim3(1024), 0, s, P_part, nblocks, E, T, P_ws, P_out,
                       status_ws, status_out);
}

int select_tokens_per_block(int E) {
    const int G = E >= 64 ? 64 : pow2_at_least(E);
    return 4 * (64 / G);
}

void launch_balance(const float* dots, int NC, const float* logit_bias, const float* noise, int gate, int T, int E,
                    int k, uint64_t seed, uint64_t noise_offset, const int32_t* topk_idx, const float* topk_gate,
                    const float* P_part, const float* P_mean, int seq_len, float* imp_part, float* load_part,
                    float* cnt_part, float* z_part, float* imp_ws, float* load_ws, float* cnt_ws, float* z_ws,
                    float* seq_part, const moe_stats* st, int k_mean, int p_row_tokens, hipStream_t s) {
    if (T <= 0) return;
    const int G = E >= 64 ? 64 : pow2_at_least(E);
    const int V = (E + G - 1) / G;
    const int nb = select_blocks(T, E);
    const bool noisy = gate == MOE_GATE_NOISY_TOPK;
#define MOE_BAL_ARGS dots, NC, logit_bias, noise, gate, T, E, k, seed, noise_offset, topk_idx, topk_gate, imp_part, load_part, cnt_part, z_part
#define MOE_BAL(GG, VV) hipLaunchKernelGGL((k_balance<GG, VV>), dim3(nb), dim3(256), 0, s, MOE_BAL_ARGS)
    if (G < 64) {
        switch (G) {
            case 1: MOE_BAL(1, 1); break;
            case 2: MOE_BAL(2, 1); break;
            case 4: MOE_BAL(4, 1); break;
            case 8: MOE_BAL(8, 1); break;
            case 16: MOE_BAL(16, 1); break;
            default: MOE_BAL(32, 1); break;
        }
    } else if (V <= 1) MOE_BAL(64, 1);
    else if (V <= 2) MOE_BAL(64, 2);
    else if (V <= 4) MOE_BAL(64, 4);
    else if (V <= 8) MOE_BAL(64, 8);
    else MOE_BAL(64, 16);
#undef MOE_BAL
#undef MOE_BAL_ARGS
    const dim3 cs((E + 63) / 64);
    hipLaunchKernelGGL(k_column_sums, cs, dim3(1024), 0, s, imp_part, nb, E, 1.0f, imp_ws, st->importance);
    if (noisy) hipLaunchKernelGGL(k_column_sums, cs, dim3(1024), 0, s, load_part, nb, E, 1.0f, load_ws, st->load);
    hipLaunchKernelGGL(k_column_sums, dim3(1), dim3(1024), 0, s, z_part, nb, 1, 1.0f / (float)T, z_ws, (float*)nullptr);
    // sequences of seq_len tokens cover whole select blocks (seq_len is a
    // multiple of 256, every block size divides 256); seq_len = 0: one
    // sequence over all blocks
    const int L = seq_len > 0 ? seq_len : T;
    const int nseq = T / L;
    const int bps = seq_len > 0 ? seq_len / select_tokens_per_block(E) : nb;
    const int pps = seq_len > 0 ? seq_len / p_row_tokens : 0;    // rows of P_part per sequence
    if (seq_len == 0)
        hipLaunchKernelGGL(k_column_sums, cs, dim3(1024), 0, s, cnt_part, nb, E, 1.0f, cnt_ws, (float*)nullptr);
    hipLaunchKernelGGL(k_seq_aux, dim3(nseq), dim3(256), 0, s, cnt_part, P_part,
                       seq_len > 0 ? (const float*)nullptr : (const float*)cnt_ws,
                       seq_len > 0 ? (const float*)nullptr : P_mean, L, k_mean, E, bps, pps, seq_part);
    hipLaunchKernelGGL(k_balance_final, dim3(1), dim3(256), 0, s, imp_ws, noisy ? load_ws : (const float*)nullptr,
                       z_ws, seq_part, nseq, E, st->importance_cv2, noisy ? st->load_cv2 : (float*)nullptr,
                       st->z_loss, st->seq_aux);
}

void launch_ec_route(const float* dots, const float* logit_bias, int T, int E, int C, float* S, float* P_ws,
                     float* P_out, int32_t* status, int32_t* status_out, int32_t* topk_idx, float* topk_gate,
                     hipStream_t s) {
    if (T > 0) {
        hipLaunchKernelGGL(k_ec_scores, dim3((T + 255) / 256), dim3(256), 0, s, dots, logit_bias, T, E, S, status);
        hipLaunchKernelGGL(k_column_sums, dim3((E + 63) / 64), dim3(1024), 0, s, S, T, E, 1.0f / (float)T, P_ws,
                           P_out);
        hipLaunchKernelGGL(k_ec_select, dim3(E), dim3(1024), 0, s, S, T, E, C, topk_idx, topk_gate);
    }
    hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, s, status, status_out);
}

void launch_update_bias(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s) {
    hipLaunchKernelGGL(k_update_bias, dim3(1), dim3(1024), 0, s, counts, E, gamma, bias);
}

void launch_zero_i32(int32_t* p, int n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_zero_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
}

}  // namespace moe
