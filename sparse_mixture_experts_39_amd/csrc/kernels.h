// Internal launchers of the gfx950 kernels (host side).  Every launcher only
// enqueues work on the given stream; argument validation happens in
// moe_api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "tile_plan.h"

namespace moe {

// route.hip
// zero_word (optional) is set to 0 by this launch, visible to later launches on the stream.
void launch_router_dots(bool bf16, const void* x, const float* w0, const float* w1, int T, int d, int E, int NC,
                        float* dots, hipStream_t s,
                        int32_t* zero_word = nullptr);
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
// g1 / g2 (optional): the scan also writes the tile plans of the two expert
// GEMMs that follow, from the kept counts (tile_plan.h).
void launch_scan(const int32_t* hist, int nblocks, int E, int64_t capacity,
                 int32_t* blockbase, int32_t* offsets, const float* P, const moe_stats* st, hipStream_t s,
                 const PlanGeom* g1 = nullptr, const PlanGeom* g2 = nullptr);
void launch_scatter(const int32_t* topk_idx, int64_t n_assign, int E, const int32_t* blockbase,
                    const int32_t* offsets, int64_t capacity, int32_t* perm_src, int32_t* slot_pos, hipStream_t s);
// Static device scratch of moe_dispatch_noalloc: its size, and its device
// address on the current device (never the symbol itself in host code).
constexpr size_t kDispatchScratchBytes = (size_t)4 << 20;
hipError_t dispatch_scratch(void** ptr);
// Scatter (slot_pos / perm_src, as launch_scatter) and the row copy x[t] ->
// x_perm[slot_pos[t][j]] for every kept slot, in one launch (two when a row
// has more than 1024 16-byte chunks or a token more than 64 slots);
// d * elem_bytes a multiple of 16.
void launch_scatter_permute(const int32_t* topk_idx, int64_t T, int k, int E, const int32_t* blockbase,
                            const int32_t* offsets, int64_t capacity, const void* x, int d, int elem_bytes,
                            int32_t* perm_src, int32_t* slot_pos, void* x_perm, hipStream_t s);

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
// epi: 0 store, 1 relu, 2 swiglu (B0 = gate, B1 = up, N = d_ff, output width N),
// 3 swiglu that also stores a | u to C2 [rows][ldc2 >= 2N], 4 relu that also
// stores a to C2.
// Builds the tile plan on the device (offsets == NULL: one group of max_rows
// rows, whose offsets go to plan_copy), then runs the GEMM and its split-K
// fixup; with 256-row bf16 tiles, a 64-row tile of the same launch covers the
// rows an expert has left past its whole tiles when there are at most 64.
// With arows != NULL row i of the grouped A is row arows[i] / arow_div of A,
// which has a_rows rows of lda elements (under 2^31 bytes).
hipError_t launch_grouped_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B0, const void* B1,
                               int64_t b_expert_stride, void* C, int64_t ldc, int N, int K, int E,
                               int64_t max_rows, const int32_t* offsets, int32_t* plan, int32_t* plan_copy,
                               float* partial, int BM, int BN, hipStream_t s, void* C2 = nullptr,
                               int64_t ldc2 = 0, bool plan_ready = false, const int32_t* arows = nullptr,
                               int64_t a_rows = 0, int arow_div = 1);
// The tile plans of two grouped GEMMs over the same expert groups in one
// launch; the GEMMs are then launched with plan_ready = true.
hipError_t launch_tile_plans(bool bf16, const int32_t* offsets, int E, int64_t max_rows, int epi1, int N1, int K1,
                             int BM1, int BN1, int32_t* plan1, int epi2, int N2, int K2, int BM2, int BN2,
                             int32_t* plan2, hipStream_t s);
GemmShape pick_gemm_shape(bool bf16, int epi, int64_t rows, int E, int N, int K = 0);
// Plan geometry of a grouped GEMM launch (as launch_grouped_gemm sets it),
// for a plan written ahead of the launch (plan_ready).
PlanGeom plan_geom(bool bf16, int epi, int N, int K, int BM, int BN, int32_t* pre);
// C[r][n] = sum_k A[r][k] B_e[k][n] over the rows r of expert e (bf16), with
// B_e read as stored ([K][N], row stride ldb): rows k < K1 from B0 + e
// bstride, the rest from B1 + e bstride (row k - K1).  The forward's grouped
// GEMM with the weight tile read by transposing LDS reads; its tile plan,
// remainder tiles and split-K tail (plan, plan_copy, partial as for
// launch_grouped_gemm).
bool grouped_gemm_nn_supported(int64_t lda, int K, int K1, int64_t ldb, int N, bool has_b1);
hipError_t launch_grouped_gemm_nn(const void* A, int64_t lda, const void* B0, const void* B1, int K1, int64_t ldb,
                                  int64_t bstride, void* C, int64_t ldc, int N, int K, int E, int64_t max_rows,
                                  const int32_t* offsets, int32_t* plan, int32_t* plan_copy, float* partial,
                                  hipStream_t s);

// backward.hip
// dst[b][c][coff + r] = src[b][r][c]; R and C multiples of 64.
void launch_transpose(const void* src, int B, int R, int C, int64_t sbatch, void* dst, int64_t ldd, int64_t dbatch,
                      int coff, int elem_bytes, hipStream_t s);
void launch_zero_f32(float* p, int64_t n, hipStream_t s);
// dy_perm[r] = gates[a] dy[a / slots] and dg[a] = <dy[a / slots], y_perm[r]>
// for every kept row r (a = perm_src[r]).
void launch_bwd_rows(bool bf16, const void* dy, const void* y_perm, const int32_t* perm_src, const int32_t* offsets,
                     int E, const float* gates, int slots, int d, int64_t max_rows, void* dy_perm, float* dg,
                     hipStream_t s);
// da | du (row stride 2F; F for ReLU) and h from dh, a, u (row stride ld_au)
// on the kept rows (offsets == NULL: the first max_rows rows).
void launch_bwd_act(bool bf16, bool swiglu, const void* dh, const void* a, const void* u, int64_t ld_au,
                    const int32_t* offsets, int E, int64_t max_rows, int F, void* dadu, void* h, hipStream_t s);
// C_e[M][N] = sum over the rows r of expert e of A[r][m] B[r][n]; max_rows
// bounds every expert's row count.
hipError_t launch_gemm_tn(bool bf16, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int M, int N,
                          int E, const int32_t* offsets, int64_t max_rows, hipStream_t s);
// C[r][n] = sum_k A[r][k] B_e[k][n] over the rows r of expert e (bf16),
// with B_e = B0 + e bstride for k < K1 and B1 + e bstride (row k - K1)
// beyond (B1 NULL: all of B0); prefix holds E + 1 ints of scratch.  Use
// only where gemm_nn_supported() holds.
// offsets = {0, rows}: one group of rows.
void launch_single_group_offsets(int32_t* offsets, int64_t rows, hipStream_t s);
bool gemm_nn_supported(int64_t max_rows, int64_t lda, int K, int K1, int64_t ldb, int N);
hipError_t launch_gemm_nn(const void* A, int64_t lda, const void* B0, const void* B1, int K1, int64_t ldb,
                          int64_t bstride, void* C, int64_t ldc, int N, int K, int E, const int32_t* offsets,
                          int64_t max_rows, int32_t* prefix, hipStream_t s);
void launch_bwd_router(const float* dots, int NC, const float* logit_bias, const int32_t* idx, const float* gates,
                       const float* dg, int gate, int T, int E, int slots, float* dz, hipStream_t s);
// idx != NULL: dz is zero outside the token's selected experts (sum over
// its slots); NULL: sum over every expert.
void launch_bwd_dx(bool bf16, const void* dy, const void* dx_perm, const int32_t* slot_pos, int slots,
                   const void* dx_shared, const float* dz, const int32_t* idx, const float* w_router, int T, int E,
                   int d, bool residual, void* dx, hipStream_t s);
int bwd_wr_chunks(int T, int E);
// dW_r = dz^T x and db = sum_t dz; part holds bwd_wr_chunks(T, E) * E * (d + 1) floats.
void launch_bwd_wr(bool bf16, const float* dz, const void* x, int T, int E, int d, float* part, float* dw, float* db,
                   hipStream_t s);

}  // namespace moe
