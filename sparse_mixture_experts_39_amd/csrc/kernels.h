// Internal launchers of the gfx950 kernels (host side).  Every launcher only
// enqueues work on the given stream; argument validation happens in
// moe_api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// route.hip
void launch_router_dots(bool bf16, const void* x, const float* w0, const float* w1, int T, int d, int E, int NC,
                        float* dots, hipStream_t s);
int select_blocks(int T, int E);
// Hierarchical gate: A groups of E / A experts, KP groups then KS experts per
// group per token; P partials of hier_select_blocks(T) blocks.
int hier_select_blocks(int T);
// Capacity reroute: assignments with slot_pos < 0 move, in order, to their
// token's best other expert with room (offsets: the capacity cut's kept
// prefix).  Rewrites idx in place.
void launch_reroute(int32_t* idx, const float* keys, const int32_t* slot_pos, const int32_t* offsets, int T, int E,
                    int k, int64_t C, hipStream_t s);
void launch_select_hier(const float* dots, int NC, const float* logit_bias, int T, int E, int A, int KP, int KS,
                        int32_t* topk_idx, float* topk_gate, float* scores, float* P_part, int32_t* status,
                        hipStream_t s);
void launch_select(const float* dots, int NC, const float* logit_bias, const float* sel_bias, const float* noise,
                   const int32_t* token_ids, int gate, int T, int E, int k, uint64_t seed, uint64_t noise_offset,
                   int32_t* topk_idx, float* topk_gate, float* scores, float* P_part, int32_t* status,
                   hipStream_t s);
void launch_reduce_P(const float* P_part, int nblocks, int E, int T, float* P_ws, float* P_out,
                     const int32_t* status_ws, int32_t* status_out, hipStream_t s);
void launch_zero_i32(int32_t* p, int n, hipStream_t s);
int select_tokens_per_block(int E);
void launch_balance(const float* dots, int NC, const float* logit_bias, const float* noise, int gate, int T, int E,
                    int k, uint64_t seed, uint64_t noise_offset, const int32_t* topk_idx, const float* topk_gate,
                    const float* P_part, const float* P_mean, int seq_len, float* imp_part, float* load_part,
                    float* cnt_part, float* z_part, float* imp_ws, float* load_ws, float* cnt_ws, float* z_ws,
                    float* seq_part, const moe_stats* st, int k_mean, int p_row_tokens, hipStream_t s);
void launch_update_bias(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s);
void launch_ec_route(const float* dots, const float* logit_bias, int T, int E, int C, float* S, float* P_ws,
                     float* P_out, int32_t* status, int32_t* status_out, int32_t* topk_idx, float* topk_gate,
                     hipStream_t s);

// dispatch.hip
constexpr int kAssignBlock = 256;  // assignments per histogram / scatter block
void launch_histogram(const int32_t* topk_idx, int64_t n_assign, int E, int32_t* hist, hipStream_t s);
void launch_scan(const int32_t* hist, int nblocks, int E, int64_t capacity,
                 int32_t* blockbase, int32_t* offsets, const float* P, const moe_stats* st, hipStream_t s);
void launch_scatter(const int32_t* topk_idx, int64_t n_assign, int E, const int32_t* blockbase,
                    const int32_t* offsets, int64_t capacity, int32_t* perm_src, int32_t* slot_pos, hipStream_t s);
void launch_permute_rows(const void* x, int k, int d, int elem_bytes, const int32_t* perm_src, const int32_t* offsets,
                         int E, int64_t max_rows, void* x_perm, hipStream_t s);

// combine.hip
void launch_combine(const void* y_perm, const int32_t* slot_pos, const float* gates, const void* residual,
                    const void* shared, void* out, int T, int d, int k, bool bf16, hipStream_t s);

// ffn.hip
struct GemmShape {
    int BM, BN;
};
size_t ffn_tile_plan_ints(int E);
// Split-K partial accumulator workspace needed by a BM x BN launch.
size_t gemm_partial_bytes(int BM, int BN);
// Grouped GEMM C[rows][N] = act(A[rows][K] . B_e[N][K]^T) per expert group.
// epi: 0 store, 1 relu, 2 swiglu (B0 = gate, B1 = up, N = d_ff, output width N).
// Builds the tile plan on the device (offsets == NULL: one group of max_rows
// rows, whose offsets go to plan_copy), then runs the GEMM and its split-K
// fixup.
hipError_t launch_grouped_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B0, const void* B1,
                               int64_t b_expert_stride, void* C, int64_t ldc, int N, int K, int E,
                               int64_t max_rows, const int32_t* offsets, int32_t* plan, int32_t* plan_copy,
                               float* partial, int BM, int BN, hipStream_t s);
GemmShape pick_gemm_shape(bool bf16, int epi, int64_t rows, int E, int N);

}  // namespace moe
