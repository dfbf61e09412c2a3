// Dispatch stage for gfx950: per-expert histogram, prefix scan with the
// capacity cut, stable scatter of assignments into expert order, and the row
// permutation of the token activations.
//
// The layer re-arranges tokens by expert, runs every expert on its batch and
// restores the token order afterwards (CS25 "Lecture29" notes, "Top-k routing
// semantics").  The order inside an expert is the assignment order
// a = t*k + j, so the permutation is the stable counting sort of the
// assignments by expert; with a capacity C (Lecture29, "Inference load
// balance": C = ceil(alpha T k / E)) the first C assignments of an expert are
// kept and later ones dropped (CS336 lecture 4 notes, section 10).  Ranks come
// from positions, never from the arrival order of atomics, so every output is
// bitwise reproducible.
//
// Kernels
//   k_histogram   256 assignments per block; lanes holding the same expert
//                 are found with one ballot per expert-id bit; per-wave counts
//                 in LDS; per-block histogram hist[b][e]
//   k_scan        one block: column scan over blocks (rank base of each block
//                 inside each expert), capacity cut, exclusive scan over
//                 experts -> offsets, and the load statistics; k_scan_wave
//                 is the same for at most 64 experts in one wave
//   k_scatter     same ranking as k_histogram, plus the wave prefix inside the
//                 block -> slot_pos / perm_src
//   k_permute_tokens  token-major: each token row of x is read once and
//                 written to the rows its kept slots point at (slot_pos),
//                 16-byte vector copies
#include "device_common.h"
#include "kernels.h"

namespace moe {

// Lanes of the wave whose (valid) expert id equals this lane's.
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid, int ebits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bm = __ballot(bit);
        m &= bit ? bm : ~bm;
    }
    return m;
}

static int id_bits(int E) { int b = 0; while ((1 << b) < E) ++b; return b; }

__global__ __launch_bounds__(256) void k_histogram(const int32_t* __restrict__ topk_idx, int64_t n_assign, int E,
                                                   int ebits, int32_t* __restrict__ hist) {
    extern __shared__ int32_t cnt[];  // [4][E]
    for (int i = threadIdx.x; i < 4 * E; i += 256) cnt[i] = 0;
    __syncthreads();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t a = (int64_t)blockIdx.x * kAssignBlock + threadIdx.x;
    const int ev = a < n_assign ? topk_idx[a] : -1;
    const bool valid = ev >= 0 && ev < E;   // an id outside [0, E) is ignored (never indexes memory)
    const int e = valid ? ev : 0;
    const uint64_t m = match_lanes(e, valid, ebits);
    if (valid && lane == __ffsll((unsigned long long)m) - 1) cnt[wave * E + e] = __popcll(m);
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += 256)
        hist[(int64_t)blockIdx.x * E + i] = ((cnt[i] + cnt[E + i]) + cnt[2 * E + i]) + cnt[3 * E + i];
}

// Column e of the per-block histogram: blockbase[b][e] = exclusive prefix over
// the blocks (16 loads in flight at a time); returns the column total.
__device__ __forceinline__ int32_t column_scan(const int32_t* __restrict__ hist, int nblocks, int E, int e,
                                               int32_t* __restrict__ blockbase) {
    int32_t run = 0;
    int b = 0;
    for (; b + 16 <= nblocks; b += 16) {
        int32_t h[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) h[u] = hist[(int64_t)(b + u) * E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            blockbase[(int64_t)(b + u) * E + e] = run;
            run += h[u];
        }
    }
    for (; b < nblocks; ++b) {
        blockbase[(int64_t)b * E + e] = run;
        run += hist[(int64_t)b * E + e];
    }
    return run;
}

__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ hist, int nblocks, int E,
                                               int64_t capacity, int32_t* __restrict__ blockbase,
                                               int32_t* __restrict__ offsets, const float* __restrict__ P,
                                               int32_t* counts_out, int32_t* kept_out, float* f_out,
                                               int32_t* dropped_out, float* imbalance_out, float* aux_out) {
    __shared__ int32_t scan[1024];
    __shared__ int64_t kept_red[1024];
    __shared__ int64_t cnt_red[1024];
    __shared__ int32_t max_red[1024];
    __shared__ double aux_red[1024];
    const int e = threadIdx.x;
    int32_t c = 0, kp = 0;
    if (e < E) {
        c = column_scan(hist, nblocks, E, e, blockbase);
        kp = (capacity >= 0 && (int64_t)c > capacity) ? (int32_t)capacity : c;
    }
    // inclusive scan of kept over experts (Hillis-Steele, integers)
    scan[e] = kp;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = e >= off ? scan[e - off] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    if (e < E) {
        offsets[e] = scan[e] - kp;
        if (e == E - 1) offsets[E] = scan[e];
        if (counts_out) counts_out[e] = c;
        if (kept_out) kept_out[e] = kp;
    }
    // integer totals: the assignments made (T k for token choice, E C for
    // expert choice), the kept ones, and the largest expert count
    kept_red[e] = kp;
    cnt_red[e] = c;
    max_red[e] = c;
    __syncthreads();
    for (int half = 512; half >= 1; half >>= 1) {
        if (e < half) {
            kept_red[e] += kept_red[e + half];
            cnt_red[e] += cnt_red[e + half];
            max_red[e] = max(max_red[e], max_red[e + half]);
        }
        __syncthreads();
    }
    const int64_t total = cnt_red[0];
    const double fe = (e < E && total > 0) ? (double)c / (double)total : 0.0;
    if (e < E && f_out) f_out[e] = (float)fe;
    // aux = E sum_e f_e P_e, fixed tree
    aux_red[e] = (e < E && P) ? fe * (double)P[e] : 0.0;
    __syncthreads();
    for (int half = 512; half >= 1; half >>= 1) {
        if (e < half) aux_red[e] += aux_red[e + half];
        __syncthreads();
    }
    if (e == 0) {
        if (dropped_out) dropped_out[0] = (int32_t)(total - kept_red[0]);
        if (imbalance_out) imbalance_out[0] = total > 0 ? (float)((double)max_red[0] * (double)E / (double)total) : 0.0f;
        if (aux_out && P) aux_out[0] = (float)((double)E * aux_red[0]);
    }
}

// k_scan for at most 64 experts: one wave, lane e = expert e, shuffles
// instead of LDS and barriers.  The sums are the same: the integer scans are
// exact, and the fixed halving tree of the aux sum differs from the wide
// kernel's only in levels that add zeros.
__global__ __launch_bounds__(64) void k_scan_wave(const int32_t* __restrict__ hist, int nblocks, int E,
                                                  int64_t capacity, int32_t* __restrict__ blockbase,
                                                  int32_t* __restrict__ offsets, const float* __restrict__ P,
                                                  int32_t* counts_out, int32_t* kept_out, float* f_out,
                                                  int32_t* dropped_out, float* imbalance_out, float* aux_out) {
    const int e = threadIdx.x;
    int32_t c = 0, kp = 0;
    if (e < E) {
        c = column_scan(hist, nblocks, E, e, blockbase);
        kp = (capacity >= 0 && (int64_t)c > capacity) ? (int32_t)capacity : c;
    }
    int32_t sc = kp;   // inclusive scan of kept over experts
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t v = __shfl_up(sc, off, 64);
        if (e >= off) sc += v;
    }
    int64_t kt = kp, ct = c;
    int32_t mx = c;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kt += __shfl_down(kt, off, 64);
        ct += __shfl_down(ct, off, 64);
        mx = max(mx, __shfl_down(mx, off, 64));
    }
    kt = __shfl(kt, 0, 64);
    ct = __shfl(ct, 0, 64);
    mx = __shfl(mx, 0, 64);
    if (e < E) {
        offsets[e] = sc - kp;
        if (e == E - 1) offsets[E] = sc;
        if (counts_out) counts_out[e] = c;
        if (kept_out) kept_out[e] = kp;
    }
    const double fe = (e < E && ct > 0) ? (double)c / (double)ct : 0.0;
    if (e < E && f_out) f_out[e] = (float)fe;
    double ax = (e < E && P) ? fe * (double)P[e] : 0.0;
#pragma unroll
    for (int half = 32; half >= 1; half >>= 1) {
        const double o = __shfl_down(ax, half, 64);
        if (e < half) ax += o;
    }
    if (e == 0) {
        if (dropped_out) dropped_out[0] = (int32_t)(ct - kt);
        if (imbalance_out) imbalance_out[0] = ct > 0 ? (float)((double)mx * (double)E / (double)ct) : 0.0f;
        if (aux_out && P) aux_out[0] = (float)((double)E * ax);
    }
}

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ topk_idx, int64_t n_assign, int E,
                                                 int ebits, const int32_t* __restrict__ blockbase,
                                                 const int32_t* __restrict__ offsets, int64_t capacity,
                                                 int32_t* __restrict__ perm_src, int32_t* __restrict__ slot_pos) {
    extern __shared__ int32_t cnt[];  // [4][E]
    for (int i = threadIdx.x; i < 4 * E; i += 256) cnt[i] = 0;
    __syncthreads();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t a = (int64_t)blockIdx.x * kAssignBlock + threadIdx.x;
    const int ev = a < n_assign ? topk_idx[a] : -1;
    const bool valid = ev >= 0 && ev < E;   // an id outside [0, E) is ignored (never indexes memory)
    const int e = valid ? ev : 0;
    const uint64_t m = match_lanes(e, valid, ebits);
    if (valid && lane == __ffsll((unsigned long long)m) - 1) cnt[wave * E + e] = __popcll(m);
    __syncthreads();
    if (!valid) {
        if (a < n_assign) slot_pos[a] = -1;
        return;
    }
    int32_t r = blockbase[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < wave; ++w) r += cnt[w * E + e];
    r += __popcll(m & ((1ull << lane) - 1ull));
    if (capacity < 0 || (int64_t)r < capacity) {
        const int32_t row = offsets[e] + r;
        slot_pos[a] = row;
        perm_src[row] = (int32_t)a;
    } else {
        slot_pos[a] = -1;
    }
}

// Grid-stride over (token, 16-byte chunk): the chunk is read once and stored
// to every kept slot's row.  A wave covers consecutive chunks of one row, so
// its slot_pos reads hit one address.
__global__ __launch_bounds__(256) void k_permute_tokens(const uint4* __restrict__ x, int k, int cpr,
                                                        const int32_t* __restrict__ slot_pos, int64_t T,
                                                        uint4* __restrict__ x_perm) {
    const int64_t total = T * cpr;
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < total; base += stride) {
        uint4 v[4];
        int64_t t[4];
        int c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            t[u] = -1;
            if (i < total) {
                t[u] = i / cpr;
                c[u] = (int)(i - t[u] * cpr);
                v[u] = x[i];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t[u] < 0) continue;
            for (int j = 0; j < k; ++j) {
                const int32_t r = slot_pos[t[u] * k + j];
                if (r >= 0) x_perm[(int64_t)r * cpr + c[u]] = v[u];
            }
        }
    }
}

void launch_histogram(const int32_t* topk_idx, int64_t n_assign, int E, int32_t* hist, hipStream_t s) {
    const int nb = (int)((n_assign + kAssignBlock - 1) / kAssignBlock);
    if (nb == 0) return;
    hipLaunchKernelGGL(k_histogram, dim3(nb), dim3(256), 4 * E * sizeof(int32_t), s, topk_idx, n_assign, E,
                       id_bits(E), hist);
}

void launch_scan(const int32_t* hist, int nblocks, int E, int64_t capacity, int32_t* blockbase,
                 int32_t* offsets, const float* P, const moe_stats* st, hipStream_t s) {
    if (E <= 64)
        hipLaunchKernelGGL(k_scan_wave, dim3(1), dim3(64), 0, s, hist, nblocks, E, capacity, blockbase, offsets, P,
                           st ? st->counts : nullptr, st ? st->kept : nullptr, st ? st->f : nullptr,
                           st ? st->n_dropped : nullptr, st ? st->imbalance : nullptr, st ? st->aux : nullptr);
    else
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, hist, nblocks, E, capacity, blockbase, offsets, P,
                           st ? st->counts : nullptr, st ? st->kept : nullptr, st ? st->f : nullptr,
                           st ? st->n_dropped : nullptr, st ? st->imbalance : nullptr, st ? st->aux : nullptr);
}

void launch_scatter(const int32_t* topk_idx, int64_t n_assign, int E, const int32_t* blockbase,
                    const int32_t* offsets, int64_t capacity, int32_t* perm_src, int32_t* slot_pos, hipStream_t s) {
    const int nb = (int)((n_assign + kAssignBlock - 1) / kAssignBlock);
    if (nb == 0) return;
    hipLaunchKernelGGL(k_scatter, dim3(nb), dim3(256), 4 * E * sizeof(int32_t), s, topk_idx, n_assign, E, id_bits(E),
                       blockbase, offsets, capacity, perm_src, slot_pos);
}

void launch_permute_tokens(const void* x, int k, int d, int elem_bytes, const int32_t* slot_pos, int64_t T,
                           void* x_perm, hipStream_t s) {
    const int cpr = d * elem_bytes / 16;
    const int64_t total = T * cpr;
    if (total == 0) return;
    int64_t nb = (total + 1023) / 1024;
    if (nb > 16384) nb = 16384;
    hipLaunchKernelGGL(k_permute_tokens, dim3((unsigned)nb), dim3(256), 0, s, (const uint4*)x, k, cpr, slot_pos, T,
                       (uint4*)x_perm);
}

}  // namespace moe
