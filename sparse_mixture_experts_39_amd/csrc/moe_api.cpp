// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout and the order of kernel launches for each stage.
// Nothing here allocates, frees or synchronizes; every check runs before the
// first launch of a call.
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include "kernels.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(const moe_config* c) { return c->act_dtype == MOE_BF16 ? 2 : 4; }
bool is_bf16(const moe_config* c) { return c->act_dtype == MOE_BF16; }
bool expert_choice(const moe_config* c) { return c->gate == MOE_GATE_EXPERT_CHOICE; }
bool hierarchical(const moe_config* c) { return c->gate == MOE_GATE_HIERARCHICAL; }
// router product columns: E logits, then E noise-scale logits (noisy gate) or
// the n_groups primary logits (hierarchical gate)
int router_cols(const moe_config* c) {
    return c->gate == MOE_GATE_NOISY_TOPK ? 2 * c->n_experts
                                          : c->n_experts + (hierarchical(c) ? c->n_groups : 0);
}
// blocks of the selection kernel (rows of the P partials)
int route_blocks(const moe_config* c) {
    if (c->T <= 0) return 0;
    return hierarchical(c) ? moe::hier_select_blocks(c->T) : moe::select_blocks(c->T, c->n_experts);
}
// selection slots per token: k, or E under expert choice
int slots_of(const moe_config* c) { return expert_choice(c) ? c->n_experts : c->top_k; }
int64_t n_assign(const moe_config* c) { return (int64_t)c->T * slots_of(c); }

// C = ceil(cf * T * k / E) with the capacity factor taken as the decimal it
// is written as: cf is read as q / 10^6, q = cf * 10^6 rounded to the nearest
// integer (halves up), and the ceiling is taken on integers, so factors such
// as 1.1 or 0.1 give the capacity of the printed formula instead of that of
// their nearest binary fraction.  At most `limit`.
int64_t decimal_capacity(double cf, int64_t T, int64_t k, int64_t E, int64_t limit) {
    const double scaled = cf * 1e6;      // own statement: never fused with the + 0.5
    const double q = floor(scaled + 0.5);
    if (!(q < 9.0e18)) return limit;
    const unsigned __int128 num = (unsigned __int128)(uint64_t)q * (uint64_t)(T * k);
    const uint64_t den = 1000000ull * (uint64_t)E;
    const unsigned __int128 C = num / den + (num % den != 0 ? 1 : 0);
    return C < (unsigned __int128)limit ? (int64_t)C : limit;
}

// tokens each expert takes under expert choice (cf <= 0 reads as 1; at most T)
int64_t ec_capacity_of(const moe_config* c) {
    const double cf = c->capacity_factor > 0.0 ? c->capacity_factor : 1.0;
    return decimal_capacity(cf, c->T, c->top_k, c->n_experts, c->T);
}

// capacity cut applied by the dispatch stage (-1: none); at most T * k, so
// it always fits in 32 bits
int64_t capacity_of(const moe_config* c) {
    if (expert_choice(c)) return -1;
    if (!(c->capacity_factor > 0.0)) return -1;
    return decimal_capacity(c->capacity_factor, c->T, c->top_k, c->n_experts, (int64_t)c->T * c->top_k);
}

int64_t max_rows_of(const moe_config* c) {
    if (expert_choice(c)) return ec_capacity_of(c) * (int64_t)c->n_experts;
    const int64_t tk = n_assign(c);
    const int64_t cap = capacity_of(c);
    if (cap < 0) return tk;
    const int64_t ec = cap * (int64_t)c->n_experts;
    return ec < tk ? ec : tk;
}

// Workspace regions (byte offsets from the workspace base).
struct Layout {
    size_t dots, P_part, P_ws, status;                    // route
    size_t hist, blockbase;                               // dispatch
    size_t H, plan_up, plan_down, plan_copy;              // experts
    size_t Hs, plan_s_up, plan_s_down, plan_s_copy;       // shared expert
    size_t idx, gates, slot_pos, perm_src, offsets;       // whole-layer intermediates
    size_t x_perm, y_perm, shared_out;
    size_t partial;                                       // split-K accumulators
    size_t imp_part, load_part, cnt_part, z_part, imp_ws, load_ws, cnt_ws, z_ws, seq_part;   // balance statistics
    size_t ec_scores;                                     // expert choice: S [T][E]
    size_t keys;                                          // capacity reroute: selection keys [T][E]
    size_t total;
};

// Split-K workspace: the largest need over the grouped GEMMs the layer runs.
size_t partial_bytes_of(const moe_config* c) {
    const bool bf = c->act_dtype == MOE_BF16;
    const int epi_up = c->act == MOE_ACT_SWIGLU ? 2 : 1;
    size_t b = 0;
    auto need = [&](int epi, int64_t rows, int E, int N, int K) {
        const moe::GemmShape g = moe::pick_gemm_shape(bf, epi, rows, E, N, K);
        const size_t n = moe::gemm_partial_bytes(g.BM, g.BN);
        if (n > b) b = n;
    };
    const int64_t R = max_rows_of(c);
    if (R > 0) {
        need(epi_up, R, c->n_experts, c->d_ff, c->d_model);
        need(0, R, c->n_experts, c->d_model, c->d_ff);
    }
    if (c->n_shared > 0 && c->T > 0) {
        need(2, c->T, 1, c->d_ff_shared, c->d_model);
        need(0, c->T, 1, c->d_model, c->d_ff_shared);
    }
    return b;
}

Layout compute_layout(const moe_config* c) {
    Layout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    const int E = c->n_experts, T = c->T;
    const int NC = router_cols(c);
    const int es = elem_bytes(c);
    const int64_t R = max_rows_of(c);
    const int64_t nasg_blocks = (n_assign(c) + moe::kAssignBlock - 1) / moe::kAssignBlock;
    const size_t plan = moe::ffn_tile_plan_ints(E) * sizeof(int32_t);
    L.dots = take((size_t)T * NC * sizeof(float));
    L.P_part = take((size_t)route_blocks(c) * E * sizeof(float));
    L.P_ws = take((size_t)E * sizeof(float));
    L.status = take(sizeof(int32_t));
    L.hist = take((size_t)nasg_blocks * E * sizeof(int32_t));
    L.blockbase = take((size_t)nasg_blocks * E * sizeof(int32_t));
    L.H = take((size_t)R * c->d_ff * es);
    L.plan_up = take(plan);
    L.plan_down = take(plan);
    L.plan_copy = take(2 * sizeof(int32_t));
    const bool sh = c->n_shared > 0;
    L.Hs = take(sh ? (size_t)T * c->d_ff_shared * es : 0);
    L.plan_s_up = take(plan);
    L.plan_s_down = take(plan);
    L.plan_s_copy = take(2 * sizeof(int32_t));
    L.idx = take((size_t)n_assign(c) * sizeof(int32_t));
    L.gates = take((size_t)n_assign(c) * sizeof(float));
    L.slot_pos = take((size_t)n_assign(c) * sizeof(int32_t));
    L.perm_src = take((size_t)R * sizeof(int32_t));
    L.offsets = take((size_t)(E + 1) * sizeof(int32_t));
    L.x_perm = take((size_t)R * c->d_model * es);
    L.y_perm = take((size_t)R * c->d_model * es);
    L.shared_out = take(sh ? (size_t)T * c->d_model * es : 0);
    L.partial = take(partial_bytes_of(c));
    const size_t sb = T > 0 ? (size_t)moe::select_blocks(T, E) : 0;
    L.imp_part = take(sb * E * sizeof(float));
    L.load_part = take(sb * E * sizeof(float));
    L.cnt_part = take(sb * E * sizeof(float));
    L.z_part = take(sb * sizeof(float));
    L.imp_ws = take((size_t)E * sizeof(float));
    L.load_ws = take((size_t)E * sizeof(float));
    L.cnt_ws = take((size_t)E * sizeof(float));
    L.z_ws = take(sizeof(float));
    L.seq_part = take((size_t)(T / 256 + 1) * sizeof(float));
    L.ec_scores = take(expert_choice(c) ? (size_t)T * E * sizeof(float) : 0);
    L.keys = take((c->flags & MOE_F_REROUTE) ? (size_t)T * E * sizeof(float) : 0);
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

moe_status hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    g_last_hip_error = (int32_t)e;
    return MOE_ERR_HIP;
}

moe_status after_launch() { return hip_status(hipGetLastError()); }

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (ws_bytes < compute_layout(c).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// ---- backward workspace ----------------------------------------------------
struct BwdLayout {
    size_t dots, dg, dz, wr_part;                                  // router
    size_t dyp, a, u, dh, dadu, hh, dxp, w2t, w13t;                // routed experts
    size_t sa, su, sdh, sdadu, shh, sdx, sw2t, sw13t;              // shared expert
    size_t plan, plan_copy, plan_s_copy, partial, nn_prefix;
    size_t total;
};

// The input-gradient products dh = dy W2 and dx = [da|du] [W1; W3] either
// run on the forward's grouped GEMM against transposed weight copies, or
// read the weights as stored (the NN product).  The copies cost a pass over
// every weight, which only pays off when each expert has many rows: the NN
// product is used below kNnRowsPerExpert rows per expert (bf16).
constexpr int64_t kNnRowsPerExpert = 512;

// bf16 backward products through the weights as stored: the grouped GEMM
// reading its weight tiles k-major (transposing LDS reads) takes dh = dy W2
// and dx = [da | du] [W1; W3] without weight copies, whatever the rows.
bool use_km_products(const moe_config* c, int F) {
    if (!is_bf16(c)) return false;
    const bool swiglu = c->act == MOE_ACT_SWIGLU;
    const int ig = swiglu ? 2 : 1, d = c->d_model;
    return moe::grouped_gemm_nn_supported(d, d, d, F, F, false) &&
           moe::grouped_gemm_nn_supported((int64_t)ig * F, ig * F, F, d, d, swiglu);
}

bool use_nn_product(const moe_config* c, int64_t rows, int E, int F) {
    if (use_km_products(c, F)) return false;
    if (!is_bf16(c) || rows <= 0 || rows >= kNnRowsPerExpert * E) return false;
    const int ig = c->act == MOE_ACT_SWIGLU ? 2 : 1;
    const int d = c->d_model;
    return moe::gemm_nn_supported(rows, d, d, d, F, F) && moe::gemm_nn_supported(rows, (int64_t)ig * F, ig * F, F, d, d);
}

bool bwd_gate_supported(const moe_config* c) {
    return c->gate == MOE_GATE_SOFTMAX_TOPK || c->gate == MOE_GATE_SOFTMAX_FULL ||
           c->gate == MOE_GATE_SIGMOID_BIAS || c->gate == MOE_GATE_EXPERT_CHOICE || c->gate == MOE_GATE_HASH;
}

// Split-K workspace of the backward's grouped GEMMs (all plain stores).
size_t bwd_partial_bytes_of(const moe_config* c) {
    const bool bf = is_bf16(c);
    size_t b = 0;
    auto need = [&](int64_t rows, int E, int N) {
        const moe::GemmShape g = moe::pick_gemm_shape(bf, 0, rows, E, N);
        const size_t n = moe::gemm_partial_bytes(g.BM, g.BN);
        if (n > b) b = n;
    };
    const int64_t R = max_rows_of(c);
    if (R > 0) {
        need(R, c->n_experts, c->d_ff);
        need(R, c->n_experts, c->d_model);
    }
    if (c->n_shared > 0 && c->T > 0) {
        need(c->T, 1, c->d_ff_shared);
        need(c->T, 1, c->d_model);
    }
    return b;
}

BwdLayout compute_bwd_layout(const moe_config* c) {
    BwdLayout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    const int E = c->n_experts, T = c->T, d = c->d_model, F = c->d_ff;
    const size_t es = (size_t)elem_bytes(c);
    const int ig = c->act == MOE_ACT_SWIGLU ? 2 : 1;
    const int64_t R = max_rows_of(c);
    L.dots = take((size_t)T * E * sizeof(float));
    L.dg = take((size_t)n_assign(c) * sizeof(float));
    L.dz = take((size_t)T * E * sizeof(float));
    L.wr_part = take((size_t)moe::bwd_wr_chunks(T, E) * E * (d + 1) * sizeof(float));
    L.dyp = take((size_t)R * d * es);
    L.a = take((size_t)R * F * es);
    L.u = take(ig == 2 ? (size_t)R * F * es : 0);
    L.dh = take((size_t)R * F * es);
    L.dadu = take((size_t)R * ig * F * es);
    L.hh = take((size_t)R * F * es);
    L.dxp = take((size_t)R * d * es);
    const bool nn = use_nn_product(c, R, E, F) || use_km_products(c, F);
    L.w2t = take(nn ? 0 : (size_t)E * F * d * es);
    L.w13t = take(nn ? 0 : (size_t)E * d * ig * F * es);
    const bool sh = c->n_shared > 0;
    const size_t Fs = sh ? (size_t)c->d_ff_shared : 0;
    L.sa = take((size_t)T * Fs * es);
    L.su = take((size_t)T * Fs * es);
    L.sdh = take((size_t)T * Fs * es);
    L.sdadu = take((size_t)T * 2 * Fs * es);
    L.shh = take((size_t)T * Fs * es);
    L.sdx = take(sh ? (size_t)T * d * es : 0);
    const bool snn = sh && (use_nn_product(c, T, 1, (int)Fs) || use_km_products(c, (int)Fs));
    L.sw2t = take(snn ? 0 : Fs * d * es);
    L.sw13t = take(snn ? 0 : (size_t)d * 2 * Fs * es);
    L.plan = take(moe::ffn_tile_plan_ints(E) * sizeof(int32_t));
    L.plan_copy = take(2 * sizeof(int32_t));
    L.plan_s_copy = take(2 * sizeof(int32_t));
    L.partial = take(bwd_partial_bytes_of(c));
    L.nn_prefix = take((size_t)(E + 1) * sizeof(int32_t));
    L.total = o;
    return L;
}

}  // namespace

extern "C" {

moe_status moe_validate_config(const moe_config* c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->T < 0 || c->d_model <= 0 || c->d_ff <= 0 || c->n_experts <= 0 || c->top_k <= 0) return MOE_ERR_INVALID_ARG;
    if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (c->act != MOE_ACT_RELU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
    if (c->gate < MOE_GATE_SOFTMAX_TOPK || c->gate > MOE_GATE_HIERARCHICAL) return MOE_ERR_INVALID_ARG;
    if (c->top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
    if (c->n_shared < 0 || c->n_shared > 1) return MOE_ERR_INVALID_ARG;
    if (c->n_shared == 1 && c->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
    if (!isfinite(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if (c->flags & ~(uint32_t)(MOE_F_ADD_RESIDUAL | MOE_F_NOISE_INPUT | MOE_F_REROUTE)) return MOE_ERR_INVALID_ARG;
    if (c->flags & MOE_F_REROUTE) {
        if (!(c->capacity_factor > 0.0) || c->gate == MOE_GATE_EXPERT_CHOICE) return MOE_ERR_INVALID_ARG;
        if (c->gate == MOE_GATE_HIERARCHICAL) return MOE_ERR_UNSUPPORTED;
    }
    if (c->top_k > 16 || c->n_experts > 1024) return MOE_ERR_UNSUPPORTED;
    if (c->d_model % 64 || c->d_ff % 64) return MOE_ERR_UNSUPPORTED;
    if (c->n_shared == 1 && (c->d_ff_shared % 64 || c->act != MOE_ACT_SWIGLU)) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)c->T * c->top_k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)c->T * slots_of(c) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (c->reserved != 0 || c->seq_len < 0) return MOE_ERR_INVALID_ARG;
    if (c->gate == MOE_GATE_HIERARCHICAL) {
        if (c->n_groups < 1 || c->group_top_k < 1 || c->group_top_k > c->n_groups ||
            c->n_experts % c->n_groups != 0 || c->top_k % c->group_top_k != 0 ||
            c->top_k / c->group_top_k > c->n_experts / c->n_groups)
            return MOE_ERR_INVALID_ARG;
        if (c->n_groups > 64 || c->n_experts / c->n_groups > 64) return MOE_ERR_UNSUPPORTED;
    } else if (c->n_groups != 0 || c->group_top_k != 0) {
        return MOE_ERR_INVALID_ARG;
    }
    if (c->seq_len > 0 && (c->seq_len % 256 != 0 || c->T % c->seq_len != 0)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int64_t moe_max_rows(const moe_config* c) {
    if (moe_validate_config(c) != MOE_OK) return -1;
    return max_rows_of(c);
}

int64_t moe_capacity(const moe_config* c) {
    if (moe_validate_config(c) != MOE_OK) return -1;
    return expert_choice(c) ? ec_capacity_of(c) : capacity_of(c);
}

int32_t moe_route_slots(const moe_config* c) {
    if (moe_validate_config(c) != MOE_OK) return -1;
    return slots_of(c);
}

moe_status moe_workspace_size(const moe_config* c, size_t* bytes) {
    const moe_status st = moe_validate_config(c);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = compute_layout(c).total;
    return MOE_OK;
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

moe_status moe_route(const moe_config* c, const void* x, const moe_weights* w, int32_t* topk_idx, float* topk_gate,
                     float* scores, const moe_stats* st, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    const bool hashed = c->gate == MOE_GATE_HASH;
    if (!w || (!hashed && !w->w_router)) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && ((!hashed && !x) || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
    if (hashed && c->T > 0 && !w->token_ids) return MOE_ERR_INVALID_ARG;
    if (hierarchical(c) && !w->w_group_router) return MOE_ERR_INVALID_ARG;
    if (c->gate == MOE_GATE_NOISY_TOPK) {
        if (!w->w_noise) return MOE_ERR_INVALID_ARG;
        if ((c->flags & MOE_F_NOISE_INPUT) && !w->noise) return MOE_ERR_INVALID_ARG;
    }
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    hipStream_t h = (hipStream_t)stream;
    const Layout L = compute_layout(c);
    const int E = c->n_experts, T = c->T;
    const bool noisy = c->gate == MOE_GATE_NOISY_TOPK;
    const int NC = router_cols(c);
    float* dots = at<float>(ws, L.dots);
    int32_t* status = at<int32_t>(ws, L.status);
    const bool balance = st && (st->z_loss || st->importance || st->importance_cv2 || st->load || st->load_cv2 ||
                                st->seq_aux);
    if ((hashed || hierarchical(c)) && balance) return MOE_ERR_UNSUPPORTED;
    // the device status word is cleared by the router product (or on its own
    // without one); the selection sets it after
    if (hashed)
        moe::launch_zero_i32(status, 1, h);
    else
        moe::launch_router_dots(is_bf16(c), x, w->w_router,
                                noisy ? w->w_noise : (hierarchical(c) ? w->w_group_router : nullptr), T, c->d_model,
                                E, NC, dots, h, status);
    if (hierarchical(c)) {
        moe::launch_select_hier(dots, NC, w->logit_bias, T, E, c->n_groups, c->group_top_k,
                                c->top_k / c->group_top_k, topk_idx, topk_gate, scores, at<float>(ws, L.P_part),
                                status, h);
        moe::launch_reduce_P(at<float>(ws, L.P_part), route_blocks(c), E, T, at<float>(ws, L.P_ws),
                             st ? st->P : nullptr, status, st ? st->device_status : nullptr, h);
        return after_launch();
    }
    if (expert_choice(c)) {
        float* S = scores ? scores : at<float>(ws, L.ec_scores);
        moe::launch_ec_route(dots, w->logit_bias, T, E, (int)ec_capacity_of(c), S, at<float>(ws, L.P_ws),
                             st ? st->P : nullptr, status, st ? st->device_status : nullptr, topk_idx, topk_gate, h);
        if (balance)
            moe::launch_balance(dots, NC, w->logit_bias, nullptr, c->gate, T, E, slots_of(c), c->seed, c->noise_offset,
                                topk_idx, topk_gate, S, at<float>(ws, L.P_ws), c->seq_len, at<float>(ws, L.imp_part),
                                at<float>(ws, L.load_part), at<float>(ws, L.cnt_part), at<float>(ws, L.z_part),
                                at<float>(ws, L.imp_ws), at<float>(ws, L.load_ws), at<float>(ws, L.cnt_ws),
                                at<float>(ws, L.z_ws), at<float>(ws, L.seq_part), st, c->top_k, 1, h);
        return after_launch();
    }
    const float* noise = (noisy && (c->flags & MOE_F_NOISE_INPUT)) ? w->noise : nullptr;
    const bool reroute = (c->flags & MOE_F_REROUTE) != 0;
    float* keys = scores ? scores : (reroute ? at<float>(ws, L.keys) : nullptr);
    moe::launch_select(dots, NC, w->logit_bias, c->gate == MOE_GATE_SIGMOID_BIAS ? w->sel_bias : nullptr, noise,
                       hashed ? w->token_ids : nullptr, c->gate, T, E, c->top_k, c->seed, c->noise_offset, topk_idx,
                       topk_gate, keys,
                       at<float>(ws, L.P_part), status, h);
    if (reroute && T > 0) {
        // the capacity cut of dispatch, on scratch buffers, then the moves
        const int64_t na = n_assign(c);
        const int nb = (int)((na + moe::kAssignBlock - 1) / moe::kAssignBlock);
        int32_t* hist = at<int32_t>(ws, L.hist);
        int32_t* bbase = at<int32_t>(ws, L.blockbase);
        int32_t* offs = at<int32_t>(ws, L.offsets);
        const int64_t cap = capacity_of(c);
        moe::launch_histogram(topk_idx, na, E, hist, h);
        moe::launch_scan(hist, nb, E, cap, bbase, offs, nullptr, nullptr, h);
        moe::launch_scatter(topk_idx, na, E, bbase, offs, cap, at<int32_t>(ws, L.perm_src),
                            at<int32_t>(ws, L.slot_pos), h);
        moe::launch_reroute(topk_idx, keys, at<int32_t>(ws, L.slot_pos), offs, T, E, c->top_k, cap, h);
    }
    moe::launch_reduce_P(at<float>(ws, L.P_part), T > 0 ? moe::select_blocks(T, E) : 0, E, T, at<float>(ws, L.P_ws),
                         st ? st->P : nullptr, status, st ? st->device_status : nullptr, h);
    if (balance)
        moe::launch_balance(dots, NC, w->logit_bias, noise, c->gate, T, E, c->top_k, c->seed, c->noise_offset,
                            topk_idx, topk_gate, at<float>(ws, L.P_part), at<float>(ws, L.P_ws), c->seq_len,
                            at<float>(ws, L.imp_part), at<float>(ws, L.load_part), at<float>(ws, L.cnt_part),
                            at<float>(ws, L.z_part), at<float>(ws, L.imp_ws), at<float>(ws, L.load_ws),
                            at<float>(ws, L.cnt_ws), at<float>(ws, L.z_ws), at<float>(ws, L.seq_part), st,
                            c->top_k, moe::select_tokens_per_block(E), h);
    return after_launch();
}

moe_status moe_update_bias(const moe_config* c, const int32_t* counts, float gamma, float* sel_bias, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (!counts || !sel_bias || !(gamma == gamma) || gamma - gamma != 0.0f) return MOE_ERR_INVALID_ARG;
    moe::launch_update_bias(counts, c->n_experts, gamma, sel_bias, (hipStream_t)stream);
    return after_launch();
}

// The dispatch kernels on validated arguments; gu / gd (optional): the scan
// also writes the tile plans of the two expert GEMMs that follow.  x_perm ==
// NULL: only the permutation (perm_src, slot_pos) is written, no rows are
// copied (the layer's up projection then gathers the rows of x itself).
static moe_status dispatch_stages(const moe_config* c, const void* x, const int32_t* topk_idx, void* x_perm,
                                  int32_t* expert_offsets, int32_t* perm_src, int32_t* slot_pos, const moe_stats* st,
                                  void* ws, hipStream_t h, const moe::PlanGeom* gu, const moe::PlanGeom* gd) {
    const Layout L = compute_layout(c);
    const int E = c->n_experts;
    const int64_t na = n_assign(c);
    const int nb = (int)((na + moe::kAssignBlock - 1) / moe::kAssignBlock);
    const int64_t cap = capacity_of(c);
    int32_t* hist = at<int32_t>(ws, L.hist);
    int32_t* bbase = at<int32_t>(ws, L.blockbase);
    const float* P = (st && st->P) ? st->P : at<float>(ws, L.P_ws);
    moe::launch_histogram(topk_idx, na, E, hist, h);
    moe::launch_scan(hist, nb, E, cap, bbase, expert_offsets, P, st, h, gu, gd);
    if (x_perm)
        moe::launch_scatter_permute(topk_idx, c->T, slots_of(c), E, bbase, expert_offsets, cap, x, c->d_model,
                                    elem_bytes(c), perm_src, slot_pos, x_perm, h);
    else
        moe::launch_scatter(topk_idx, na, E, bbase, expert_offsets, cap, perm_src, slot_pos, h);
    return after_launch();
}

moe_status moe_dispatch(const moe_config* c, const void* x, const int32_t* topk_idx, void* x_perm,
                        int32_t* expert_offsets, int32_t* perm_src, int32_t* slot_pos, const moe_stats* st, void* ws,
                        size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (!expert_offsets) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!x || !topk_idx || !x_perm || !perm_src || !slot_pos)) return MOE_ERR_INVALID_ARG;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    return dispatch_stages(c, x, topk_idx, x_perm, expert_offsets, perm_src, slot_pos, st, ws, (hipStream_t)stream,
                           nullptr, nullptr);
}

moe_status moe_dispatch_noalloc(const moe_config* c, const void* x, const int32_t* topk_idx, void* x_perm,
                                int32_t* expert_offsets, int32_t* perm_src, int32_t* slot_pos, const moe_stats* st,
                                void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (!expert_offsets) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!x || !topk_idx || !x_perm || !perm_src || !slot_pos)) return MOE_ERR_INVALID_ARG;
    const int E = c->n_experts;
    const int64_t na = n_assign(c);
    const int nb = (int)((na + moe::kAssignBlock - 1) / moe::kAssignBlock);
    const size_t hist_bytes = align_up((size_t)nb * E * sizeof(int32_t));
    if (2 * hist_bytes > moe::kDispatchScratchBytes) return MOE_ERR_UNSUPPORTED;
    void* base = nullptr;
    if ((s = hip_status(moe::dispatch_scratch(&base))) != MOE_OK) return s;
    hipStream_t h = (hipStream_t)stream;
    int32_t* hist = (int32_t*)base;
    int32_t* bbase = (int32_t*)((char*)base + hist_bytes);
    const int64_t cap = capacity_of(c);
    const float* P = (st && st->P) ? st->P : nullptr;   // aux needs the caller's P
    moe::launch_histogram(topk_idx, na, E, hist, h);
    moe::launch_scan(hist, nb, E, cap, bbase, expert_offsets, P, st, h);
    moe::launch_scatter_permute(topk_idx, c->T, slots_of(c), E, bbase, expert_offsets, cap, x, c->d_model,
                                elem_bytes(c), perm_src, slot_pos, x_perm, h);
    return after_launch();
}

// One grouped GEMM of an expert stack (tile plan, GEMM and split-K fixup, all
// on the device).  up = true: a -> H (ReLU / SwiGLU epilogue); up = false:
// H -> y.  With offsets == NULL the call covers one group of `rows` rows (the
// shared expert) and the plan writes its offsets to plan_copy.
// Epilogue and tile shape of one of the two products (the same for its tile
// plan and its launch).
static int gemm_epi(const moe_config* c, bool up, bool pre) {
    const bool swiglu = c->act == MOE_ACT_SWIGLU;
    return up ? (swiglu ? (pre ? 3 : 2) : (pre ? 4 : 1)) : 0;
}
static moe::GemmShape gemm_shape(const moe_config* c, bool up, bool pre, int64_t rows, int E, int F) {
    return moe::pick_gemm_shape(is_bf16(c), gemm_epi(c, up, pre), rows, E, up ? F : c->d_model, up ? c->d_model : F);
}

// up with arows != NULL: row i of the up projection's input is row
// arows[i] / slots of a (the T rows of x; arows holds assignment ids).
static moe_status run_gemm(const moe_config* c, bool up, const void* a, int64_t rows, int E, const int32_t* offsets,
                           const void* w1, const void* w3, const void* w2, int F, void* dst, int32_t* plan,
                           int32_t* plan_copy, float* partial, hipStream_t h, void* pre = nullptr,
                           bool plan_ready = false, const int32_t* arows = nullptr) {
    const bool bf = is_bf16(c);
    const int d = c->d_model;
    const bool swiglu = c->act == MOE_ACT_SWIGLU;
    // up with pre != NULL: the epilogue also stores the pre-activations
    const int epi = gemm_epi(c, up, pre != nullptr);
    const moe::GemmShape g = gemm_shape(c, up, pre != nullptr, rows, E, F);
    const hipError_t e = up ? moe::launch_grouped_gemm(bf, epi, a, d, w1, w3, (int64_t)F * d, dst, F, F, d, E, rows,
                                                       offsets, plan, plan_copy, partial, g.BM, g.BN, h, pre,
                                                       (int64_t)(swiglu ? 2 : 1) * F, plan_ready, arows, c->T,
                                                       slots_of(c))
                            : moe::launch_grouped_gemm(bf, 0, a, F, w2, nullptr, (int64_t)d * F, dst, d, d, F, E,
                                                       rows, offsets, plan, plan_copy, partial, g.BM, g.BN, h,
                                                       nullptr, 0, plan_ready);
    if (e != hipSuccess) return hip_status(e);
    return after_launch();
}

static moe_status check_ffn_args(const moe_config* c, const void* a, const int32_t* offsets, const moe_weights* w,
                                 const void* dst, bool need_up, bool need_down) {
    if (!w || !offsets) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!a || !dst)) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && need_up && (!w->w_gate || (c->act == MOE_ACT_SWIGLU && !w->w_up))) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && need_down && !w->w_down) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status moe_expert_up(const moe_config* c, const void* x_perm, const int32_t* expert_offsets, const moe_weights* w,
                         void* hbuf, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if ((s = check_ffn_args(c, x_perm, expert_offsets, w, hbuf, true, false)) != MOE_OK) return s;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    const int64_t R = max_rows_of(c);
    if (R == 0) return MOE_OK;
    const Layout L = compute_layout(c);
    return run_gemm(c, true, x_perm, R, c->n_experts, expert_offsets, w->w_gate, w->w_up, nullptr, c->d_ff, hbuf,
                    at<int32_t>(ws, L.plan_up), at<int32_t>(ws, L.plan_copy), at<float>(ws, L.partial),
                    (hipStream_t)stream);
}

moe_status moe_expert_up_train(const moe_config* c, const void* x_perm, const int32_t* expert_offsets,
                               const moe_weights* w, void* hbuf, void* pre_act, void* ws, size_t ws_bytes,
                               void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if ((s = check_ffn_args(c, x_perm, expert_offsets, w, hbuf, true, false)) != MOE_OK) return s;
    if (c->T > 0 && !pre_act) return MOE_ERR_INVALID_ARG;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    const int64_t R = max_rows_of(c);
    if (R == 0) return MOE_OK;
    const Layout L = compute_layout(c);
    return run_gemm(c, true, x_perm, R, c->n_experts, expert_offsets, w->w_gate, w->w_up, nullptr, c->d_ff, hbuf,
                    at<int32_t>(ws, L.plan_up), at<int32_t>(ws, L.plan_copy), at<float>(ws, L.partial),
                    (hipStream_t)stream, pre_act);
}

moe_status moe_expert_down(const moe_config* c, const void* hbuf, const int32_t* expert_offsets, const moe_weights* w,
                           void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if ((s = check_ffn_args(c, hbuf, expert_offsets, w, y_perm, false, true)) != MOE_OK) return s;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    const int64_t R = max_rows_of(c);
    if (R == 0) return MOE_OK;
    const Layout L = compute_layout(c);
    return run_gemm(c, false, hbuf, R, c->n_experts, expert_offsets, nullptr, nullptr, w->w_down, c->d_ff, y_perm,
                    at<int32_t>(ws, L.plan_down), at<int32_t>(ws, L.plan_copy), at<float>(ws, L.partial),
                    (hipStream_t)stream);
}

// Tile plan geometry of the two expert GEMMs (up, down) of the layer, the
// plans going to the workspace's plan_up / plan_down.
static void ffn_plan_geoms(const moe_config* c, void* ws, moe::PlanGeom* gu, moe::PlanGeom* gd) {
    const Layout L = compute_layout(c);
    const int64_t R = max_rows_of(c);
    const bool bf = is_bf16(c);
    const int E = c->n_experts, d = c->d_model, F = c->d_ff;
    const moe::GemmShape su = gemm_shape(c, true, false, R, E, F);
    const moe::GemmShape sd = gemm_shape(c, false, false, R, E, F);
    *gu = moe::plan_geom(bf, gemm_epi(c, true, false), F, d, su.BM, su.BN, at<int32_t>(ws, L.plan_up));
    *gd = moe::plan_geom(bf, 0, d, F, sd.BM, sd.BN, at<int32_t>(ws, L.plan_down));
}

// The expert FFN on validated arguments; plans_ready: the dispatch scan has
// already written both tile plans; arows != NULL: x_perm is x and row i of
// the experts' input is its row arows[i] / slots (arows: perm_src).
static moe_status ffn_stages(const moe_config* c, const void* x_perm, const int32_t* expert_offsets,
                             const moe_weights* w, void* y_perm, void* ws, hipStream_t h, bool plans_ready,
                             const int32_t* arows = nullptr) {
    const int64_t R = max_rows_of(c);
    if (R == 0) return MOE_OK;
    const Layout L = compute_layout(c);
    void* H = at<void>(ws, L.H);
    const bool bf = is_bf16(c);
    const int E = c->n_experts, d = c->d_model, F = c->d_ff;
    int32_t* pu = at<int32_t>(ws, L.plan_up);
    int32_t* pd = at<int32_t>(ws, L.plan_down);
    int32_t* pc = at<int32_t>(ws, L.plan_copy);
    float* part = at<float>(ws, L.partial);
    moe_status s;
    if (!plans_ready) {
        // both tile plans in one launch, then the two products
        const moe::GemmShape gu = gemm_shape(c, true, false, R, E, F);
        const moe::GemmShape gd = gemm_shape(c, false, false, R, E, F);
        const hipError_t e = moe::launch_tile_plans(bf, expert_offsets, E, R, gemm_epi(c, true, false), F, d, gu.BM,
                                                    gu.BN, pu, 0, d, F, gd.BM, gd.BN, pd, h);
        if (e != hipSuccess) return hip_status(e);
    }
    if ((s = run_gemm(c, true, x_perm, R, E, expert_offsets, w->w_gate, w->w_up, nullptr, F, H, pu, pc, part, h,
                      nullptr, true, arows)) != MOE_OK)
        return s;
    return run_gemm(c, false, H, R, E, expert_offsets, nullptr, nullptr, w->w_down, F, y_perm, pd, pc, part, h,
                    nullptr, true);
}

moe_status moe_expert_ffn(const moe_config* c, const void* x_perm, const int32_t* expert_offsets,
                          const moe_weights* w, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if ((s = check_ffn_args(c, x_perm, expert_offsets, w, y_perm, true, true)) != MOE_OK) return s;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    return ffn_stages(c, x_perm, expert_offsets, w, y_perm, ws, (hipStream_t)stream, false);
}

moe_status moe_shared_expert(const moe_config* c, const void* x, const moe_weights* w, void* shared_out, void* ws,
                             size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (c->n_shared != 1) return MOE_ERR_INVALID_ARG;
    if (!w) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!x || !shared_out || !w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    if (c->T == 0) return MOE_OK;
    const Layout L = compute_layout(c);
    hipStream_t h = (hipStream_t)stream;
    void* Hs = at<void>(ws, L.Hs);
    if ((s = run_gemm(c, true, x, c->T, 1, nullptr, w->ws_gate, w->ws_up, nullptr, c->d_ff_shared, Hs,
                      at<int32_t>(ws, L.plan_s_up), at<int32_t>(ws, L.plan_s_copy), at<float>(ws, L.partial), h)) !=
        MOE_OK)
        return s;
    return run_gemm(c, false, Hs, c->T, 1, nullptr, nullptr, nullptr, w->ws_down, c->d_ff_shared, shared_out,
                    at<int32_t>(ws, L.plan_s_down), at<int32_t>(ws, L.plan_s_copy), at<float>(ws, L.partial), h);
}

moe_status moe_combine(const moe_config* c, const void* y_perm, const int32_t* slot_pos, const float* topk_gate,
                       const void* residual, const void* shared_out, void* out, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (c->T > 0 && (!slot_pos || !topk_gate || !out)) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && max_rows_of(c) > 0 && !y_perm) return MOE_ERR_INVALID_ARG;
    moe::launch_combine(y_perm, slot_pos, topk_gate, residual, shared_out, out, c->T, c->d_model, slots_of(c),
                        is_bf16(c), (hipStream_t)stream);
    return after_launch();
}

moe_status moe_layer_forward(const moe_config* c, const moe_weights* w, const void* x, void* out,
                             const moe_stats* st, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (!w || (c->gate != MOE_GATE_HASH && !w->w_router)) return MOE_ERR_INVALID_ARG;
    if (hierarchical(c) && !w->w_group_router) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!x || !out)) return MOE_ERR_INVALID_ARG;
    if (c->T > 0 && (!w->w_gate || !w->w_down || (c->act == MOE_ACT_SWIGLU && !w->w_up))) return MOE_ERR_INVALID_ARG;
    if (c->n_shared == 1 && c->T > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
    if (c->gate == MOE_GATE_NOISY_TOPK &&
        (!w->w_noise || ((c->flags & MOE_F_NOISE_INPUT) && !w->noise)))
        return MOE_ERR_INVALID_ARG;
    if ((s = check_ws(c, ws, ws_bytes)) != MOE_OK) return s;
    const Layout L = compute_layout(c);
    int32_t* idx = at<int32_t>(ws, L.idx);
    float* gates = at<float>(ws, L.gates);
    int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
    int32_t* perm_src = at<int32_t>(ws, L.perm_src);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    void* x_perm = at<void>(ws, L.x_perm);
    void* y_perm = at<void>(ws, L.y_perm);
    void* shared_out = c->n_shared ? at<void>(ws, L.shared_out) : nullptr;
    if ((s = moe_route(c, x, w, idx, gates, nullptr, st, ws, ws_bytes, stream)) != MOE_OK) return s;
    // the dispatch scan also writes the expert GEMMs' tile plans (one launch
    // fewer), and when x is under 2 GiB the up projection gathers its rows of
    // x through perm_src, so the dispatch copies no rows
    moe::PlanGeom gu, gd;
    ffn_plan_geoms(c, ws, &gu, &gd);
    const bool gather = (int64_t)c->T * c->d_model * elem_bytes(c) < ((int64_t)1 << 31);
    if ((s = dispatch_stages(c, x, idx, gather ? nullptr : x_perm, offsets, perm_src, slot_pos, st, ws,
                             (hipStream_t)stream, &gu, &gd)) != MOE_OK)
        return s;
    if ((s = ffn_stages(c, gather ? x : x_perm, offsets, w, y_perm, ws, (hipStream_t)stream, true,
                        gather ? perm_src : nullptr)) != MOE_OK)
        return s;
    if (shared_out && (s = moe_shared_expert(c, x, w, shared_out, ws, ws_bytes, stream)) != MOE_OK) return s;
    const void* resid = (c->flags & MOE_F_ADD_RESIDUAL) ? x : nullptr;
    return moe_combine(c, y_perm, slot_pos, gates, resid, shared_out, out, stream);
}

moe_status moe_backward_workspace_size(const moe_config* c, size_t* bytes) {
    const moe_status st = moe_validate_config(c);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = compute_bwd_layout(c).total;
    return MOE_OK;
}

}  // extern "C"

namespace {

// C[rows][N] = A[rows][K] . B_e[N][K]^T per expert group (plain store).
moe_status bwd_gemm(bool bf, const void* A, int64_t lda, const void* B, int64_t bstride, void* C, int64_t ldc, int N,
                    int K, int E, int64_t rows, const int32_t* offsets, const BwdLayout& L, void* ws,
                    int32_t* plan_copy, hipStream_t h) {
    const moe::GemmShape g = moe::pick_gemm_shape(bf, 0, rows, E, N);
    const hipError_t e = moe::launch_grouped_gemm(bf, 0, A, lda, B, nullptr, bstride, C, ldc, N, K, E, rows, offsets,
                                                  at<int32_t>(ws, L.plan), plan_copy, at<float>(ws, L.partial), g.BM,
                                                  g.BN, h);
    return e == hipSuccess ? after_launch() : hip_status(e);
}

// Backward of one expert stack over ragged row groups (offsets, or one group
// of `rows` rows when offsets is NULL; its offsets then go to plan_copy):
// X [rows][d] inputs, DY [rows][d] output gradients, W1/W3 [E][F][d],
// W2 [E][d][F].  Writes DX [rows][d] and, when dW1 is not NULL, the weight
// gradients.  Buffers: A, U, DH, HH [rows][F], DADU [rows][ig F], W2T
// [E][F][d], W13T [E][d][ig F].
struct ExpertBufs {
    void *a, *u, *dh, *dadu, *hh, *w2t, *w13t;
};

moe_status expert_backward(const moe_config* c, const void* X, const void* DY, int64_t rows, int E,
                           const int32_t* offsets, const void* W1, const void* W3, const void* W2, int F,
                           const ExpertBufs& b, void* DX, void* dW1, void* dW3, void* dW2, const BwdLayout& L,
                           void* ws, int32_t* plan_copy, hipStream_t h, const void* pre = nullptr) {
    const bool bf = is_bf16(c);
    const bool swiglu = c->act == MOE_ACT_SWIGLU;
    const int ig = swiglu ? 2 : 1;
    const int d = c->d_model;
    const int es = elem_bytes(c);
    moe_status s;
    const bool km = use_km_products(c, F);
    const bool nn = !km && use_nn_product(c, rows, E, F);
    int32_t* nn_prefix = at<int32_t>(ws, L.nn_prefix);
    // weight copies with the other dimension contiguous (only for the
    // grouped-GEMM route on copies): W2^T [E][F][d] and [W1^T | W3^T] [E][d][ig F]
    if (!nn && !km) {
        moe::launch_transpose(W2, E, d, F, (int64_t)d * F, b.w2t, d, (int64_t)F * d, 0, es, h);
        moe::launch_transpose(W1, E, F, d, (int64_t)F * d, b.w13t, (int64_t)ig * F, (int64_t)d * ig * F, 0, es, h);
        if (swiglu)
            moe::launch_transpose(W3, E, F, d, (int64_t)F * d, b.w13t, (int64_t)ig * F, (int64_t)d * ig * F, F, es,
                                  h);
    }
    // a = X W1^T and u = X W3^T: saved by the forward (pre = [a | u], row
    // stride ig F; routed experts only), else recomputed.  dh = DY W2.  The
    // first GEMM also builds the offsets of a single group.
    const void* A_ = b.a;
    const void* U_ = b.u;
    int64_t ld_au = F;
    if (pre) {
        A_ = pre;
        U_ = (const uint8_t*)pre + (size_t)F * es;
        ld_au = (int64_t)ig * F;
    } else {
        if ((s = bwd_gemm(bf, X, d, W1, (int64_t)F * d, b.a, F, F, d, E, rows, offsets, L, ws, plan_copy, h)) !=
            MOE_OK)
            return s;
        if (swiglu && (s = bwd_gemm(bf, X, d, W3, (int64_t)F * d, b.u, F, F, d, E, rows, offsets, L, ws, plan_copy,
                                    h)) != MOE_OK)
            return s;
    }
    const int32_t* offs = offsets ? offsets : plan_copy;
    int32_t* plan = at<int32_t>(ws, L.plan);
    float* partial = at<float>(ws, L.partial);
    if (km) {
        // with offsets == NULL the plan launch also writes the group's offsets
        const hipError_t e2 = moe::launch_grouped_gemm_nn(DY, d, W2, nullptr, d, F, (int64_t)d * F, b.dh, F, F, d, E,
                                                          rows, offsets, plan, plan_copy, partial, h);
        if (e2 != hipSuccess) return hip_status(e2);
    } else if (nn) {
        // a single group needs its offsets before the NN product reads them
        if (!offsets) moe::launch_single_group_offsets(plan_copy, rows, h);
        const hipError_t e2 = moe::launch_gemm_nn(DY, d, W2, nullptr, d, F, (int64_t)d * F, b.dh, F, F, d, E, offs,
                                                  rows, nn_prefix, h);
        if (e2 != hipSuccess) return hip_status(e2);
    } else if ((s = bwd_gemm(bf, DY, d, b.w2t, (int64_t)F * d, b.dh, F, F, d, E, rows, offsets, L, ws, plan_copy,
                             h)) != MOE_OK) {
        return s;
    }
    moe::launch_bwd_act(bf, swiglu, b.dh, A_, U_, ld_au, offs, offsets ? E : 1, rows, F, b.dadu, b.hh, h);
    // DX = da W1 + du W3 as one product over the concatenated reduction
    if (km) {
        const hipError_t e2 = moe::launch_grouped_gemm_nn(b.dadu, (int64_t)ig * F, W1, swiglu ? W3 : nullptr, F, d,
                                                          (int64_t)F * d, DX, d, d, ig * F, E, rows, offsets, plan,
                                                          plan_copy, partial, h);
        if (e2 != hipSuccess) return hip_status(e2);
    } else if (nn) {
        const hipError_t e2 = moe::launch_gemm_nn(b.dadu, (int64_t)ig * F, W1, swiglu ? W3 : nullptr, F, d,
                                                  (int64_t)F * d, DX, d, d, ig * F, E, offs, rows, nn_prefix, h);
        if (e2 != hipSuccess) return hip_status(e2);
    } else if ((s = bwd_gemm(bf, b.dadu, (int64_t)ig * F, b.w13t, (int64_t)d * ig * F, DX, d, d, ig * F, E, rows,
                             offsets, L, ws, plan_copy, h)) != MOE_OK) {
        return s;
    }
    if (!dW1) return MOE_OK;
    hipError_t e;
    const int Eg = offsets ? E : 1;
    if ((e = moe::launch_gemm_tn(bf, DY, d, b.hh, F, dW2, d, F, Eg, offs, rows, h)) != hipSuccess)
        return hip_status(e);
    if ((e = moe::launch_gemm_tn(bf, b.dadu, (int64_t)ig * F, X, d, dW1, F, d, Eg, offs, rows, h)) != hipSuccess)
        return hip_status(e);
    if (swiglu && (e = moe::launch_gemm_tn(bf, (const uint8_t*)b.dadu + (size_t)F * es, (int64_t)ig * F, X, d, dW3, F,
                                           d, Eg, offs, rows, h)) != hipSuccess)
        return hip_status(e);
    return after_launch();
}

}  // namespace

extern "C" {

moe_status moe_layer_backward(const moe_config* c, const moe_weights* w, const void* x, const void* dy,
                              const moe_saved* sv, const moe_grads* g, void* ws, size_t ws_bytes, void* stream) {
    moe_status s = moe_validate_config(c);
    if (s != MOE_OK) return s;
    if (!bwd_gate_supported(c) || (c->flags & MOE_F_REROUTE)) return MOE_ERR_UNSUPPORTED;
    if (!w || !sv || !g) return MOE_ERR_INVALID_ARG;
    const bool hashed = c->gate == MOE_GATE_HASH;
    const bool swiglu = c->act == MOE_ACT_SWIGLU;
    const int T = c->T, E = c->n_experts, d = c->d_model;
    const int64_t R = max_rows_of(c);
    if (!hashed && !w->w_router) return MOE_ERR_INVALID_ARG;
    // the router gradient reads 512-token chunks of x with 32-bit byte offsets
    if (!hashed && (int64_t)512 * d * 4 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!sv->expert_offsets) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!x || !dy || !g->dx || !sv->topk_idx || !sv->topk_gate || !sv->slot_pos)) return MOE_ERR_INVALID_ARG;
    if (R > 0 && (!sv->perm_src || !sv->x_perm || !sv->y_perm)) return MOE_ERR_INVALID_ARG;
    if (!w->w_gate || !w->w_down || (swiglu && !w->w_up)) return MOE_ERR_INVALID_ARG;
    const bool want_w = g->dw_gate || g->dw_up || g->dw_down;
    if (want_w && (!g->dw_gate || !g->dw_down || (swiglu != (g->dw_up != nullptr)))) return MOE_ERR_INVALID_ARG;
    const bool want_ws = g->dws_gate || g->dws_up || g->dws_down;
    if (want_ws && (c->n_shared != 1 || !g->dws_gate || !g->dws_up || !g->dws_down)) return MOE_ERR_INVALID_ARG;
    if (c->n_shared == 1 && T > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
    if (!ws) return MOE_ERR_WORKSPACE;
    const BwdLayout L = compute_bwd_layout(c);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t h = (hipStream_t)stream;
    const bool bf = is_bf16(c);
    const int ns = slots_of(c);
    float* dg = at<float>(ws, L.dg);
    float* dz = hashed ? nullptr : at<float>(ws, L.dz);

    // output-side rows: dy_r = g dY_t and the gate gradients
    moe::launch_zero_f32(dg, n_assign(c), h);
    moe::launch_bwd_rows(bf, dy, sv->y_perm, sv->perm_src, sv->expert_offsets, E, sv->topk_gate, ns, d, R,
                         at<void>(ws, L.dyp), dg, h);
    // routed experts
    if (R > 0) {
        const ExpertBufs b{at<void>(ws, L.a), at<void>(ws, L.u), at<void>(ws, L.dh), at<void>(ws, L.dadu),
                           at<void>(ws, L.hh), at<void>(ws, L.w2t), at<void>(ws, L.w13t)};
        if ((s = expert_backward(c, sv->x_perm, at<void>(ws, L.dyp), R, E, sv->expert_offsets, w->w_gate, w->w_up,
                                 w->w_down, c->d_ff, b, at<void>(ws, L.dxp), want_w ? g->dw_gate : nullptr,
                                 g->dw_up, g->dw_down, L, ws, at<int32_t>(ws, L.plan_copy), h, sv->pre_act)) !=
            MOE_OK)
            return s;
    } else if (want_w) {
        hipError_t e;
        if ((e = moe::launch_gemm_tn(bf, nullptr, d, nullptr, c->d_ff, g->dw_down, d, c->d_ff, E,
                                     sv->expert_offsets, 0, h)) != hipSuccess ||
            (e = moe::launch_gemm_tn(bf, nullptr, c->d_ff, nullptr, d, g->dw_gate, c->d_ff, d, E,
                                     sv->expert_offsets, 0, h)) != hipSuccess ||
            (swiglu && (e = moe::launch_gemm_tn(bf, nullptr, c->d_ff, nullptr, d, g->dw_up, c->d_ff, d, E,
                                                sv->expert_offsets, 0, h)) != hipSuccess))
            return hip_status(e);
    }
    // shared expert: every token, gate 1
    const bool sh = c->n_shared == 1 && T > 0;
    if (sh) {
        const ExpertBufs b{at<void>(ws, L.sa), at<void>(ws, L.su), at<void>(ws, L.sdh), at<void>(ws, L.sdadu),
                           at<void>(ws, L.shh), at<void>(ws, L.sw2t), at<void>(ws, L.sw13t)};
        if ((s = expert_backward(c, x, dy, T, 1, nullptr, w->ws_gate, w->ws_up, w->ws_down, c->d_ff_shared, b,
                                 at<void>(ws, L.sdx), want_ws ? g->dws_gate : nullptr, g->dws_up, g->dws_down, L, ws,
                                 at<int32_t>(ws, L.plan_s_copy), h)) != MOE_OK)
            return s;
    }
    // router: logits as the forward forms them, then dz and its products
    if (!hashed && T > 0) {
        float* dots = at<float>(ws, L.dots);
        moe::launch_router_dots(bf, x, w->w_router, nullptr, T, d, E, E, dots, h);
        moe::launch_bwd_router(dots, E, w->logit_bias, sv->topk_idx, sv->topk_gate, dg, c->gate, T, E, ns, dz, h);
    }
    if (g->dw_router || g->dlogit_bias) {
        if (hashed || T == 0) {
            if (g->dw_router) moe::launch_zero_f32(g->dw_router, (int64_t)E * d, h);
            if (g->dlogit_bias) moe::launch_zero_f32(g->dlogit_bias, E, h);
        } else {
            moe::launch_bwd_wr(bf, dz, x, T, E, d, at<float>(ws, L.wr_part), g->dw_router, g->dlogit_bias, h);
        }
    }
    // dz vanishes off the selected experts for the softmax-over-selected and
    // sigmoid gates (not for the full softmax and expert choice)
    const bool sparse_dz = c->gate == MOE_GATE_SOFTMAX_TOPK || c->gate == MOE_GATE_SIGMOID_BIAS;
    moe::launch_bwd_dx(bf, dy, at<void>(ws, L.dxp), sv->slot_pos, ns, sh ? at<void>(ws, L.sdx) : nullptr, dz,
                       sparse_dz ? sv->topk_idx : nullptr, hashed ? nullptr : w->w_router, T, E, d,
                       (c->flags & MOE_F_ADD_RESIDUAL) != 0, g->dx, h);
    return after_launch();
}

}  // extern "C"
