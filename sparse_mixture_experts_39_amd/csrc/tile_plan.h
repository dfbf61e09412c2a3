// Work decomposition of the grouped GEMM, shared by the GEMM launches
// (ffn.hip) and the dispatch scan (dispatch.hip), which can write the tile
// plans of the two expert GEMMs that follow it in the layer.
//
// Plan of one GEMM over E expert groups (2E + 5 ints): pre[0 .. E] the
// prefix over experts of whole BM-row tiles, pre[E+1 .. E+3] the split-K
// decision {full, split, tail}, pre[E+4 .. 2E+4] the prefix of remainder
// tiles.  An expert with M rows has ceil(M / BM) whole tiles, or, with
// remainder tiles enabled and r = M mod BM in 1 .. kRemThr, floor(M / BM)
// whole tiles and ceil(r / kRemBM) remainder tiles.  When the last round of
// tiles would leave the chip mostly idle (tiles mod kSplitUnits <=
// kSplitUnits / 2), those `tail` tiles are cut into `split` K ranges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kSplitUnits = 256;   // CUs of the target chip
constexpr int kMaxSplit = 16;
constexpr int kRemBM = 64;
constexpr int kRemThr = 64;    // one remainder tile at most: each re-reads its weight panel

__host__ __device__ __forceinline__ int whole_tiles(int M, int BM, bool rem) {
    const int r = M % BM;
    return (rem && r > 0 && r <= kRemThr) ? M / BM : (M + BM - 1) / BM;
}

__host__ __device__ __forceinline__ int remainder_tiles(int M, int BM, bool rem) {
    const int r = M - whole_tiles(M, BM, rem) * BM;   // 0 unless rem
    return r > 0 ? (r + kRemBM - 1) / kRemBM : 0;
}

// Split-K decision for `total` tiles of nk K slices (at least 4 slices per
// range): split ranges for each of the last `tail` tiles, or split = 1.
__host__ __device__ __forceinline__ void split_rule(int total, int nk, int& split, int& tail) {
    const int left = total % kSplitUnits;
    split = 1;
    tail = 0;
    if (left > 0 && left <= kSplitUnits / 2) {
        int sp = kSplitUnits / left;
        sp = sp < kMaxSplit ? sp : kMaxSplit;
        sp = sp < nk / 4 ? sp : nk / 4;
        if (sp >= 2) {
            split = sp;
            tail = left;
        }
    }
}

// Geometry of one GEMM's plan; pre == NULL: no plan wanted.
struct PlanGeom {
    int BM, rem, NT, nk;
    int32_t* pre;
};

}  // namespace moe
