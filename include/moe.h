/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse token-choice MoE FFN layer.
 *
 * One call of the layer, on one GPU that holds every expert, computes
 *   route -> dispatch -> expert FFNs -> combine
 * in the order the pages state the layer (CS25 "Lecture29" notes, section
 * "Top-two routing", minimal pseudocode: router logits, top-k, gates from the
 * selected logits, dispatch by expert, run the selected experts, combine and
 * restore the token order; awesome-ai-roadmap ch. 19, section 19.3.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor argument is a DEVICE pointer to memory the caller
 * owns (e.g. a PyTorch allocation).  The library never allocates, frees or
 * synchronizes: all work is enqueued on `stream` (a hipStream_t; NULL means
 * the null stream) and completes asynchronously.  No entry point copies
 * device data to the host, so a sequence of calls can be captured in a HIP
 * graph.  The library keeps no state between calls and is re-entrant; calls
 * that share a workspace must not overlap in time.
 *
 * Layouts.  Row-major, densely packed.  Activations x, x_perm, y_perm and out
 * are [rows][d_model] in the activation dtype (fp32, or bf16 stored as
 * uint16).  Expert weights use the [out][in] layout so the reduction
 * dimension is contiguous: w_gate / w_up are [E][d_ff][d_model], w_down is
 * [E][d_model][d_ff].  Router-side tensors are always fp32.  Index tensors are
 * int32.  An assignment is the pair (token t, slot j) with flat id
 * a = t * top_k + j; slots are ordered by selection score, best first.
 *
 * Errors.  Every argument check runs on the host before anything is
 * enqueued; a failed check returns MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED
 * or MOE_ERR_WORKSPACE and enqueues nothing.  A failed kernel launch returns
 * MOE_ERR_HIP; the HIP error code is kept per thread and read with
 * moe_last_hip_error().  Conditions found on the device (a non-finite
 * selection score) are reported through stats.device_status.  The library
 * never aborts and never throws across this ABI.
 *
 * Limits.  1 <= top_k <= min(n_experts, 16); n_experts <= 1024;
 * d_model and d_ff (and d_ff_shared) multiples of 64; T >= 0 and
 * T * top_k < 2^31.  n_shared is 0 or 1.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* a null required pointer, a size out of range, an unknown enum */
    MOE_ERR_UNSUPPORTED = 2,  /* a valid layer this library does not implement (alignment, limits) */
    MOE_ERR_WORKSPACE = 3,    /* workspace null or smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4           /* a HIP launch failed; see moe_last_hip_error() */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gate families (how the selection is turned into mixing weights). */
typedef enum {
    /* g = softmax over the k selected logits (Lecture29, eq. for g_i). */
    MOE_GATE_SOFTMAX_TOPK = 0,
    /* g = full softmax over all E logits, read at the selected experts, no
     * renormalisation (CS336 lecture 4 notes, section 5 listing; Switch
     * lesson: the chosen expert's output times the router probability). */
    MOE_GATE_SOFTMAX_FULL = 1,
    /* Shazeer noisy top-k: H = z + n * softplus(x W_noise), n ~ N(0,1);
     * g = softmax over the k selected H (Outrageously Large Neural Networks
     * reading notes, section 2.2). */
    MOE_GATE_NOISY_TOPK = 2,
    /* DeepSeek-V3: s = sigmoid(z); select the top-k of s + b; g = s of the
     * selected experts renormalised to sum to 1; the bias never enters g
     * (awesome-ai-roadmap 19.3.4; CS336 notes, section 12). */
    MOE_GATE_SIGMOID_BIAS = 3,
    /* Expert choice: every expert takes the C tokens with the largest router
     * probability S = softmax over the experts of z (ties to the lower token
     * index), C = ceil(cf * T * k / E) (cf <= 0 means 1; at most T), so all
     * experts get exactly C tokens and a token is taken by 0..E experts; the
     * gate of a taken (t, e) is S[t, e] (CS336 notes, section 4: top-K along
     * the rows; awesome-ai-roadmap 19.6.1).  top_k is the mean number of
     * experts per token.  The routing outputs then have E slots per token
     * (moe_route_slots): topk_idx[t][e] = e or -1, topk_gate[t][e] = S or 0. */
    MOE_GATE_EXPERT_CHOICE = 4,
    /* Hash routing: no learned score decides; a token goes to experts fixed
     * by a hash of its id, so equal tokens always meet the same experts
     * (CS336 notes, section 4, hash routing).  The key of expert e for a
     * token with id u is the top 24 bits of element i = u*E + e of the
     * Philox4x32-10 stream (counter (i>>2, noise_offset), key seed, word
     * i & 3), read as an integer; the k experts with the largest keys are
     * taken (ties to the lower index) and each gets gate 1: their outputs are
     * added (CS336 notes, section 4: some implementations add the expert
     * outputs directly).  Reads moe_weights.token_ids, not the router; P is
     * the selection frequency 1/k per taken expert, scores are the keys.
     * The balance statistics are not defined for it (no logits). */
    MOE_GATE_HASH = 5,
    /* Hierarchical (two-level) gating (Shazeer notes, appendix B: a primary
     * gate picks groups, a secondary gate picks experts inside each picked
     * group, which cuts the branching factor from n to about sqrt(n)): the
     * E experts form n_groups groups of b = E / n_groups consecutive experts;
     * the primary logits zp = W_group x pick the group_top_k largest groups,
     * the secondary logits z = W_r x (+ logit bias) of each picked group pick
     * its ks = top_k / group_top_k largest experts (ties to the lower index);
     * each gate is a softmax over the picked logits, and expert (i, j) gets
     * gp_i * gs_ij.  Slots are ordered by group rank, then expert rank.  The
     * router probability of expert (i, j) is softmax(zp)_i times the softmax
     * of group i's b logits at j.  n_groups <= 64, b <= 64; balance
     * statistics are not offered for it. */
    MOE_GATE_HIERARCHICAL = 6
} moe_gate;

/* Expert MLP: y = W2 relu(W1 a) (Shazeer notes 2.2), or
 * y = W2 (SiLU(W1 a) * W3 a) with W1 = gate, W3 = up, W2 = down (Lecture29,
 * "Dense baseline", SwiGLU MLP). */
typedef enum { MOE_ACT_RELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

enum {
    MOE_F_ADD_RESIDUAL = 1u, /* out += x (CS336 notes section 5 listing: h = sum g FFN(u) + u) */
    MOE_F_NOISE_INPUT = 2u,  /* NOISY_TOPK: read n from the caller's noise tensor
                                instead of the built-in Philox4x32-10 stream */
    /* Capacity reroute instead of drop (Lecture29, "Inference load balance":
     * an expert over capacity may drop, reroute or delay the extra tokens).
     * moe_route rewrites topk_idx: the assignments are taken in (t, j) order,
     * the first C of an expert stay, and every later one, in that order,
     * moves to its token's best other expert (largest selection key, ties to
     * the lower index) that the token does not hold yet and that still has
     * room; with none it stays and moe_dispatch drops it.  The slot keeps its
     * gate.  Needs a capacity factor > 0; not for EXPERT_CHOICE (no overflow)
     * nor HIERARCHICAL (a move would leave the picked groups). */
    MOE_F_REROUTE = 4u
};

enum { MOE_DEV_NONFINITE = 1 }; /* device_status bit: a selection score was NaN or infinite */

typedef struct {
    int32_t T;              /* tokens in this call */
    int32_t d_model;
    int32_t d_ff;           /* routed expert hidden width */
    int32_t n_experts;      /* E */
    int32_t top_k;          /* k */
    int32_t n_shared;       /* 0 or 1 always-on shared expert (SwiGLU), weight 1 */
    int32_t d_ff_shared;
    int32_t act_dtype;      /* moe_dtype of x, out, expert weights and intermediates */
    int32_t act;            /* moe_act */
    int32_t gate;           /* moe_gate */
    double capacity_factor; /* > 0: C = ceil(cf * T * k / E) with cf read as a decimal of six
                               places (q / 10^6, q = cf * 10^6 rounded, halves up) and the ceiling
                               taken exactly, at most T * k; <= 0: dropless; must be finite */
    uint32_t flags;         /* MOE_F_* */
    uint64_t seed;          /* Philox key of the noisy gate */
    uint64_t noise_offset;  /* Philox counter offset (words 2,3) of the noisy gate */
    int32_t seq_len;        /* tokens per sequence for stats.seq_aux: 0 = the whole call is one
                               sequence, else a multiple of 256 that divides T */
    int32_t reserved;       /* must be 0 */
    int32_t n_groups;       /* HIERARCHICAL: groups of the primary gate; else 0 */
    int32_t group_top_k;    /* HIERARCHICAL: groups picked per token (divides top_k); else 0 */
} moe_config;

/* Weights of one layer (device pointers). */
typedef struct {
    const float* w_router;   /* [E][d] fp32 router matrix W_r */
    const float* logit_bias; /* [E] fp32 added to the logits, or NULL */
    const float* sel_bias;   /* [E] fp32 selection-only bias (SIGMOID_BIAS), or NULL */
    const float* w_noise;    /* [E][d] fp32 noise-scale matrix (NOISY_TOPK) */
    const float* noise;      /* [T][E] fp32 standard-normal draws when MOE_F_NOISE_INPUT */
    const void* w_gate;      /* [E][d_ff][d] W1 (gate for SwiGLU, the hidden layer for ReLU) */
    const void* w_up;        /* [E][d_ff][d] W3 (SwiGLU only; NULL for ReLU) */
    const void* w_down;      /* [E][d][d_ff] W2 */
    const void* ws_gate;     /* shared expert [d_ff_shared][d] (n_shared = 1) */
    const void* ws_up;       /* shared expert [d_ff_shared][d] */
    const void* ws_down;     /* shared expert [d][d_ff_shared] */
    const int32_t* token_ids; /* [T] token ids (HASH only), else NULL */
    const float* w_group_router; /* [n_groups][d] fp32 primary router (HIERARCHICAL only) */
} moe_weights;

/* Load statistics (device pointers; any member may be NULL to skip it).
 * f_i is the fraction of the assignments (T*k; E*C under expert choice)
 * routed to expert i before capacity drops (so sum f = 1), and P_i the
 * batch mean of the router
 * probability of expert i (awesome-ai-roadmap 19.3.3; CS336 notes section
 * 9); the router probability vector is softmax(z) for the softmax gates,
 * softmax(H) for the noisy gate, s / sum(s) for the sigmoid gate and the
 * scores S for expert choice.
 * imbalance = max_i n_i / (sum_i n_i / E) (Lecture29, "Myth 3");
 * aux = E * sum_i f_i P_i (the Switch balance term without its coefficient). */
typedef struct {
    int32_t* counts;        /* [E] assignments per expert before drops */
    int32_t* kept;          /* [E] assignments kept after the capacity cut */
    float* f;               /* [E] */
    float* P;               /* [E] */
    int32_t* n_dropped;     /* [1] */
    float* imbalance;       /* [1] */
    float* aux;             /* [1] */
    int32_t* device_status; /* [1] MOE_DEV_* bits, written by moe_route */
    /* Balance and stability statistics, written by moe_route when any of
     * them is requested (all fp32, fixed summation orders):
     * z_loss = mean over tokens of (log sum_e exp z_t,e)^2 over the clean
     *   router logits, the router z-loss (CS336 notes section 11;
     *   awesome-ai-roadmap 19.6.2 table);
     * importance_e = sum over tokens of the gate expert e receives, and its
     *   CV^2 = Var / mean^2 over the experts (population variance)
     *   (Shazeer notes, Importance and CV);
     * load_e = sum_t Phi((z_t,e - kth_excluding(H_t, k, e)) / softplus((x W_noise)_t,e)),
     *   the smooth load estimate of the noisy gate, and its CV^2 (Shazeer
     *   notes, Load(X) and eq. 9); NOISY_TOPK only, untouched otherwise;
     * seq_aux = mean over sequences of seq_len tokens of E sum_e f_e P_e
     *   counted within the sequence (CS336 notes section 9: V3's
     *   complementary sequence-level balance term; awesome-ai-roadmap
     *   19.3.4). */
    float* z_loss;          /* [1] */
    float* importance;      /* [E] */
    float* importance_cv2;  /* [1] */
    float* load;            /* [E] */
    float* load_cv2;        /* [1] */
    float* seq_aux;         /* [1] */
} moe_stats;

/* ---- pure host helpers (no device work, usable without a GPU) ---------- */

/* Check a configuration.  MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED. */
moe_status moe_validate_config(const moe_config* cfg);

/* Bytes of workspace moe_layer_forward needs (the stage calls need no more). */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Rows of x_perm / y_perm the caller must allocate: T*k when dropless, else
 * min(T*k, E*C); E*C under expert choice.  -1 for an invalid configuration. */
int64_t moe_max_rows(const moe_config* cfg);

/* Expert capacity C = ceil(capacity_factor * T * k / E) (Lecture29,
 * "Inference load balance"; awesome-ai-roadmap 19.6.1 "Expert capacity"),
 * with the factor read as the six-place decimal q / 10^6 (q = factor * 10^6
 * rounded to the nearest integer, halves up) and the ceiling taken in exact
 * integer arithmetic, so 1.1 * 2560 / 64 gives 44, not 45.  Clamped to T * k
 * (to T under expert choice, where it is the tokens each expert takes).
 * -1 when dropless or invalid. */
int64_t moe_capacity(const moe_config* cfg);

/* Selection slots per token in topk_idx / topk_gate / slot_pos: top_k, or
 * n_experts under expert choice.  -1 for an invalid configuration. */
int32_t moe_route_slots(const moe_config* cfg);

/* HIP error code of the last MOE_ERR_HIP on this thread (0 if none). */
int32_t moe_last_hip_error(void);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* ---- stages ------------------------------------------------------------- */

/* Route (CS25 "Lecture29" notes, "Top-two routing": logits z = W_r x, the
 * top-k experts, gates from the selected logits; awesome-ai-roadmap 19.3.2:
 * the selected softmax equals the full softmax restricted to the top-k and
 * renormalised; CS336 lecture 4 notes, section 11: the router runs in fp32).
 * For every token: fp32 logits z = W_r x (+ logit_bias) with the
 * fixed sequential-fma order, the selection score, the k best experts
 * (score descending, ties to the lower index), the gates, and the router
 * probabilities, whose batch mean is written to stats->P.
 *   x        [T][d] act dtype          w_router [E][d] fp32
 *   topk_idx [T][k] int32 (out)        topk_gate [T][k] fp32 (out)
 *   scores   [T][E] fp32 selection scores (out, optional, may be NULL)
 * Sets stats->device_status.  Needs ws (>= moe_workspace_size bytes). */
moe_status moe_route(const moe_config* cfg, const void* x, const moe_weights* w,
                     int32_t* topk_idx, float* topk_gate, float* scores,
                     const moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Dispatch.  Per-expert histogram of the assignments, a prefix scan into
 * expert_offsets, the capacity cut, and a permutation of token rows into
 * expert-contiguous order, stable in assignment order (Lecture29, "Top-k
 * routing semantics"); with a capacity the first C assignments of each
 * expert are kept and the rest dropped (CS336 notes section 10; Switch
 * lesson token-drop answer).
 *   x [T][d] act dtype; topk_idx [T][k]
 *   x_perm [max_rows][d] act dtype (out): row r holds x[perm_src[r] / k]
 *   expert_offsets [E+1] (out): expert e owns rows [off[e], off[e+1])
 *   perm_src [max_rows] (out): assignment id of each kept row
 *   slot_pos [T][k] (out): row of each assignment, -1 if dropped
 * Writes stats counts, kept, n_dropped, f, imbalance and aux (the last two
 * read stats->P written by moe_route; pass the same stats). */
moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        void* x_perm, int32_t* expert_offsets, int32_t* perm_src,
                        int32_t* slot_pos, const moe_stats* stats,
                        void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * HIP-graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same outputs as moe_dispatch, but the per-block
 * histograms and rank bases live in a static device array of the library
 * (4 MiB per GPU, held until the process ends) instead of a caller
 * workspace, and nothing is allocated.  Needs twice ceil(T slots / 256) * E * 4
 * bytes (each rounded up to 256) of that array, i.e. ceil(T slots / 256) * E
 * up to about 524288;
 * a larger call returns MOE_ERR_UNSUPPORTED before anything is enqueued.  The
 * aux statistic reads stats->P (NULL: aux is not written).  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (several
 * streams or threads) race and must be serialised by the caller.  A failure
 * to resolve the array's device address returns MOE_ERR_HIP. */
moe_status moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx, void* x_perm,
                                int32_t* expert_offsets, int32_t* perm_src, int32_t* slot_pos,
                                const moe_stats* stats, void* stream);

/* Expert FFNs (Lecture29, "Top-two routing": run each selected expert on
 * the tokens dispatched to it; "Dense baseline": the SwiGLU MLP; Shazeer
 * notes 2.2: the one-hidden-layer ReLU expert; CS336 lecture 4 notes,
 * section 10: the tokens of all experts on one device become large matrix
 * products) as two grouped GEMMs over ragged per-expert row ranges:
 * rows [off[e], off[e+1]) of x_perm go through expert e, the hidden tensor
 * is stored in the act dtype inside ws, and y_perm receives the expert
 * outputs in the same row order (fp32 accumulation).
 *   x_perm, y_perm [max_rows][d]; expert_offsets [E+1] from moe_dispatch. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                          const moe_weights* w, void* y_perm,
                          void* ws, size_t ws_bytes, void* stream);

/* The two grouped GEMMs of moe_expert_ffn as separate calls.
 * moe_expert_up:   h[r] = SiLU(x_perm[r] W1_e^T) * (x_perm[r] W3_e^T)   (SwiGLU)
 *                  h[r] = relu(x_perm[r] W1_e^T)                        (ReLU)
 *                  for every row r of expert e; h is [max_rows][d_ff] in the act dtype.
 * moe_expert_down: y_perm[r] = h[r] W2_e^T.
 * Same layouts and ownership as moe_expert_ffn; h is caller-owned here. */
moe_status moe_expert_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                         const moe_weights* w, void* h, void* ws, size_t ws_bytes, void* stream);
/* moe_expert_up for training: also stores the pre-activations
 * pre_act[r] = [a | u] (SwiGLU, a = x_perm[r] W1_e^T, u = x_perm[r] W3_e^T,
 * row stride 2 d_ff) or a (ReLU, row stride d_ff), in the act dtype, from
 * the same fp32 accumulators as h.  moe_layer_backward reads them (through
 * moe_saved.pre_act) instead of recomputing the two products. */
moe_status moe_expert_up_train(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                               const moe_weights* w, void* h, void* pre_act, void* ws, size_t ws_bytes,
                               void* stream);
moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                           const moe_weights* w, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* The always-on shared expert on every token (awesome-ai-roadmap 19.5):
 * shared_out[T][d] = SwiGLU_shared(x).  Requires n_shared = 1. */
moe_status moe_shared_expert(const moe_config* cfg, const void* x, const moe_weights* w,
                             void* shared_out, void* ws, size_t ws_bytes, void* stream);

/* Combine.  out[t] = (residual ? x[t] : 0) + (shared_out ? shared_out[t] : 0)
 *                    + sum_j topk_gate[t][j] * y_perm[slot_pos[t][j]],
 * accumulated in fp32 in slot order, a dropped slot contributing nothing
 * (Lecture29, eq. y = sum_i g_i Expert_i; CS336 notes section 10: a dropped
 * token's MLP output is zero and the residual passes through).  One writer
 * per output element, no atomics: bitwise deterministic.
 *   residual: x [T][d] or NULL; shared_out [T][d] or NULL; out [T][d]. */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_pos,
                       const float* topk_gate, const void* residual, const void* shared_out,
                       void* out, void* stream);

/* Auxiliary-loss-free balancing step (CS336 notes section 9: after each
 * batch an underloaded expert's bias goes up by gamma and an overloaded one's
 * down; awesome-ai-roadmap 19.3.4: the bias corrects only the scores used for
 * selection).  For every expert e:
 *   sel_bias[e] += gamma * sign(mean - counts[e]),  mean = sum_e counts[e] / E,
 * with the comparison done exactly in integers (counts[e] * E vs the sum).
 * counts: [E] int32 device (e.g. stats.counts of the last call); sel_bias:
 * [E] fp32 device, updated in place.  Returns MOE_ERR_INVALID_ARG for NULL
 * pointers or a non-finite gamma. */
moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma, float* sel_bias, void* stream);

/* The whole layer (Lecture29, "Top-two routing" minimal pseudocode: route,
 * dispatch by expert, run the experts, combine and restore the token order;
 * y = sum over the selected experts of g_i Expert_i(x); awesome-ai-roadmap
 * 19.3.2 and 19.5 for the shared expert): route, dispatch, experts (+ shared
 * expert), combine, with every intermediate carved from ws.  x [T][d], out [T][d].  The residual is
 * added when cfg->flags has MOE_F_ADD_RESIDUAL.  When x is under 2 GiB the
 * dispatch writes only the permutation and the up projection reads each
 * expert row straight from x (row perm_src[r] / k), so the workspace's x_perm
 * is not written; the outputs are the same as those of the stage calls. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const void* x, void* out,
                             const moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* ---- backward --------------------------------------------------------- */

/* Tensors of the forward call that the backward reads (device pointers, as
 * the stage calls wrote them: moe_route, moe_dispatch, moe_expert_ffn). */
typedef struct {
    const int32_t* topk_idx;        /* [T][slots] */
    const float* topk_gate;         /* [T][slots] */
    const int32_t* expert_offsets;  /* [E+1] */
    const int32_t* perm_src;        /* [max_rows] */
    const int32_t* slot_pos;        /* [T][slots] */
    const void* x_perm;             /* [max_rows][d] act dtype */
    const void* y_perm;             /* [max_rows][d] act dtype: expert outputs before the gate */
    const void* pre_act;            /* [max_rows][2 d_ff] (a | u; ReLU: [max_rows][d_ff], a) act dtype from
                                       moe_expert_up_train, or NULL: the backward then recomputes a and u */
} moe_saved;

/* Gradient outputs (device pointers).  dx is required; every other member
 * may be NULL to skip it, except that dw_gate / dw_up / dw_down go together
 * (dw_up NULL for ReLU), as do dws_gate / dws_up / dws_down.  Each output is
 * overwritten, not accumulated into.  Expert weight gradients have the
 * layouts and the act dtype of the weights; router gradients are fp32. */
typedef struct {
    void* dx;            /* [T][d] act dtype */
    float* dw_router;    /* [E][d] */
    float* dlogit_bias;  /* [E] */
    void* dw_gate;       /* [E][d_ff][d]  (W1) */
    void* dw_up;         /* [E][d_ff][d]  (W3, SwiGLU) */
    void* dw_down;       /* [E][d][d_ff]  (W2) */
    void* dws_gate;      /* [d_ff_shared][d] */
    void* dws_up;        /* [d_ff_shared][d] */
    void* dws_down;      /* [d][d_ff_shared] */
} moe_grads;

/* Bytes of workspace moe_layer_backward needs. */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);

/* Backward of the whole layer for the output gradient dy [T][d] (act
 * dtype): ordinary backpropagation through the experts each token was sent
 * to, the selection held constant (Shazeer et al. reading notes, section 2.1
 * key points: a masked expert has probability and gradient exactly zero, the
 * kept ones pass a nonzero gradient to the router matrix; CS25 "Lecture29"
 * notes, Q&A "Gradient flow and training cost"; Switch Transformers lesson:
 * a single expert still trains the router through the gate probability).
 * With h, a = W1 x, u = W3 x as in moe_expert_up:
 *   dy_r  = g_tj dY_t for the row r of a kept slot (t, j);
 *   dg_tj = <dY_t, y_r> (0 for a dropped slot);
 *   dh = dy_r W2; da = dh u s (1 + a (1 - s)), s = sigmoid(a), du = dh SiLU(a)
 *   (ReLU: da = dh [a > 0]); dx_r = da W1 + du W3;
 *   dW2_e = sum_r dy_r^T h_r, dW1_e = sum_r da_r^T x_r, dW3_e = sum_r du_r^T x_r;
 *   dz from dg by the gate family: softmax over the selected logits
 *   dz_i = g_i (dg_i - sum_j g_j dg_j); full softmax and expert choice
 *   dz = p (dp - <p, dp>); sigmoid with selection bias
 *   dz_i = (dg_i - sum_j g_j dg_j) s_i (1 - s_i) / sum_sel s (the bias gets
 *   nothing); hash routing: none;
 *   dW_r = sum_t dz_t x_t^T, dlogit_bias = sum_t dz_t;
 *   dx_t = [residual] dY_t + sum_j dx_{r(t,j)} + shared expert + dz_t W_r.
 * Supported gates: SOFTMAX_TOPK, SOFTMAX_FULL, SIGMOID_BIAS, EXPERT_CHOICE,
 * HASH; the others and MOE_F_REROUTE return MOE_ERR_UNSUPPORTED, as does a
 * router gradient with d_model >= 2^20 (its 512-token chunks of x are
 * addressed with 32-bit byte offsets).  All sums
 * are fp32 in fixed orders (bitwise reproducible); intermediates (dy_r, a,
 * u, dh, da, du, h, dx_r) are stored in the act dtype.
 *   x [T][d]: the forward input; w: the forward weights; sv: the saved
 *   forward tensors; g: outputs; ws >= moe_backward_workspace_size bytes. */
moe_status moe_layer_backward(const moe_config* cfg, const moe_weights* w, const void* x, const void* dy,
                              const moe_saved* sv, const moe_grads* g, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
