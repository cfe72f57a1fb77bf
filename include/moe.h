/*
 * moe.h -- C ABI of the MI355X (gfx950) fused mixture-of-experts forward.
 *
 * The layer routes each token to top_k of num_experts expert MLPs and sums
 * their outputs with the routing weights:
 *
 *   (ids, w)  = route(router_logits_t)                        moe_topk
 *   rows      = tokens grouped expert by expert               moe_align_permute
 *   act_r     = silu(x W1_e^T) * (x W3_e^T)                   moe_grouped_gemm_w13_act
 *   out_t     = sum_k w_{t,k} * act_{r(t,k)} W2_{e}^T          moe_grouped_gemm_w2_combine
 *             (+ shared expert MLP with weight 1)
 *
 * Sources of the operation (three web pages):
 *   vLLM API docs page "vllm.model_executor.layers.fused_moe.layer",
 *     class FusedMoE: constructor arguments (num_experts, top_k, hidden_size,
 *     intermediate_size, renormalize, use_grouped_topk, num_expert_group,
 *     topk_group, scoring_func, routed_scaling_factor,
 *     e_score_correction_bias, activation "silu", is_act_and_mul),
 *     select_experts, forward_native, _load_w13 / _load_w2 (weight layout);
 *   SGLang page "srt/layers/moe/fused_moe_triton/layer.py", class FusedMoE:
 *     forward / forward_impl (dispatch -> run_moe_core -> combine);
 *   SGLang page "srt/models/deepseek_v2.py": MoEGate (fp32 router logits,
 *     fp32 correction bias), DeepseekV2MoE (grouped top-k arguments, shared
 *     expert added unscaled, routed output scaled by routed_scaling_factor,
 *     quantise-once of the input to per-token-group-128 fp8),
 *     DeepseekV2MLP (gate_up -> SiluAndMul -> down, fp8 block [128, 128]).
 *
 * Conventions for every call
 *   - Every pointer argument is DEVICE memory unless marked "host".  The
 *     caller owns all buffers; the library never allocates in a call.
 *   - All arrays are dense row-major, except the expert weight matrices
 *     (w13, w2, shared_w13, shared_w2), which the GEMM calls take in the
 *     packed layout written by moe_pack_weights; moe_params.weight_layout
 *     must say so (MOE_LAYOUT_PACKED), so that a caller handing over the
 *     pages' row-major tensors gets an error, not a wrong result.
 *     bf16 = IEEE binary32 upper half; fp8 = OCP e4m3 ("e4m3fn", max 448)
 *     stored one byte per value.
 *     Weight block scales stay row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Calls only enqueue work: no host synchronisation, no allocation, so a
 *     sequence of calls may be captured into a HIP graph.
 *   - Inputs are read-only; outputs never alias inputs (no in-place mode).
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is enqueued and a negative status is returned.
 *   - num_tokens == 0 is valid: the call returns MOE_OK and launches nothing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = -1,     /* bad shape, parameter or NULL pointer        */
    MOE_ERR_UNSUPPORTED = -2, /* valid but not built: dtype combination etc. */
    MOE_ERR_WORKSPACE = -3,   /* workspace smaller than required             */
    MOE_ERR_HIP = -4          /* a HIP launch failed                         */
};

/* Router scoring (FusedMoE scoring_func). */
enum { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 };

/* Element types. */
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_FP8_E4M3 = 2 };

/* Storage layout of the expert weight matrices handed to the GEMM calls and
 * moe_forward.  ROW_MAJOR (the pages' [N, K] tensors as loaded, and the value
 * of a zero-initialised moe_params) is rejected by those calls with
 * MOE_ERR_UNSUPPORTED; they read PACKED weights, written by moe_pack_weights
 * once at load time. */
enum { MOE_LAYOUT_ROW_MAJOR = 0, MOE_LAYOUT_PACKED = 1 };

/* Layer description (host struct, read during the call only).
 *
 * Supported (act_dtype, weight_dtype, out_dtype):
 *   (F32, F32, F32), (BF16, BF16, BF16), (BF16, FP8_E4M3, BF16).
 * fp8 weights carry one fp32 dequantisation scale per 128 x 128 block of each
 * [N, K] weight matrix (w ~= code * scale); fp8 layers quantise the input
 * and the SiLU-and-mul output per (row, group of 128) with
 * scale = max(amax, 1e-10) / 448, code = e4m3(x / scale), in fp32.
 */
typedef struct moe_params {
    int64_t num_tokens;          /* T >= 0                                     */
    int32_t num_experts;         /* E, 1..512                                  */
    int32_t top_k;               /* K, 1..min(E, 32)                           */
    int32_t hidden_size;         /* H, multiple of 64 (of 128 for fp8)         */
    int32_t intermediate_size;   /* I, multiple of 64 (of 128 for fp8)         */
    int32_t scoring_func;        /* MOE_SCORING_*                              */
    int32_t renormalize;         /* 1: weights / sum of the K selected scores  */
    int32_t num_expert_group;    /* G; 0 or 1 = ungrouped; else E % G == 0     */
    int32_t topk_group;          /* TG, 1..G, with K <= TG * E / G             */
    float routed_scaling_factor; /* multiplies every routed weight (1.0)       */
    int32_t act_dtype;           /* dtype of hidden                            */
    int32_t weight_dtype;        /* dtype of w13 / w2                          */
    int32_t out_dtype;           /* dtype of out                               */
    int32_t num_shared_experts;  /* 0, or 1: a shared expert (same format as  */
                                 /* the routed ones) of intermediate size Is  */
                                 /* (shared_intermediate) added to every      */
                                 /* token with weight 1                       */
    /* Activation variants; all zero gives the plain SiLU-and-mul layer.
     * Passages: FusedMoE is_act_and_mul and apply_router_weight_on_input
     * (vLLM page), is_gated, gemm1_alpha and gemm1_clamp_limit (SGLang layer
     * page), DeepseekV2MLP swiglu_limit with the clipped SwiGLU (SGLang
     * deepseek_v2 page).  With silu_a(z) = z * sigmoid(a * z):              */
    int32_t non_gated;           /* 0: w13 is [E, 2I, H] (gate; up) and       */
                                 /*    act = silu_a(min(g, L)) * clamp(u, -L, L) */
                                 /* 1: w13 is [E, I, H] and act = silu_a(h)   */
                                 /*    (bf16/fp32 layers)                     */
    float swiglu_alpha;          /* a; 0 means 1 (plain SiLU); >= 0          */
    float swiglu_limit;          /* L; 0 means no clamp; >= 0, gated only     */
    int32_t router_weight_on_input; /* 1: the routing weight scales the      */
                                 /* expert input, out_t = sum_k MLP(w_k x_t) */
                                 /* (+ shared MLP(x_t)); bf16/fp32 layers     */
    /* Layout of w13 / w2 / shared_w13 / shared_w2 (MOE_LAYOUT_*); the GEMM
     * calls and moe_forward require MOE_LAYOUT_PACKED. */
    int32_t weight_layout;
    /* Is, intermediate size of the shared expert; 0 means I.  Passage:
     * DeepseekV2MoE (SGLang deepseek_v2 page) builds the shared MLP with
     * moe_intermediate_size * n_shared_experts, so Is = m * I with m in
     * 1..16 (other sizes: MOE_ERR_UNSUPPORTED).  Needs num_shared_experts =
     * 1 (else it must be 0). */
    int32_t shared_intermediate;
} moe_params;

/* Bytes of device workspace that moe_forward needs for `p` (the decomposed
 * calls need no more than this).  Returns 0 for invalid parameters. */
size_t moe_workspace_size(const moe_params *p);

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(int status);

/* Weight re-layout, done once when the weights are loaded.  Each of
 * `matrices` row-major matrices of `rows` rows x `row_bytes` bytes (an
 * expert's [2I, H] gate/up or [H, I] down matrix, any element type) is
 * rewritten as [rows/16][row_bytes/64][16][64]: the 64-byte pieces of 16
 * consecutive rows that share a k range become one contiguous KiB, which is
 * the unit the GEMM kernels fetch.  Element values are copied bit for bit.
 * Not a step of the pages' method: a storage layout of this library.
 *   src  [matrices, rows, row_bytes] bytes, row-major.
 *   dst  same size, packed out; must not overlap src.
 * Errors: MOE_ERR_INVALID for negative sizes, rows % 16 != 0,
 * row_bytes % 64 != 0, NULL pointers with a non-empty size, src or dst not
 * 16-byte aligned, overlap. */
int moe_pack_weights(const void *src, void *dst, int64_t matrices, int64_t rows,
                     int64_t row_bytes, void *stream);

/* Router gate logits, the step ahead of moe_topk: logits = hidden W_g^T.
 * Passage: MoEGate (SGLang deepseek_v2 page): weight [n_routed_experts,
 * hidden_size] in the model dtype or fp32; forward is F.linear of the fp32
 * hidden for an fp32 gate, a bf16 GEMM with fp32 output for a bf16 gate.
 *   hidden        [T, H] act dtype (bf16 or fp32).
 *   gate_w        [E, H] row-major (not packed), gate_dtype MOE_DTYPE_BF16 or
 *                 MOE_DTYPE_F32.
 *   router_logits [T, E] fp32 out.  Accumulation in fp32; a bf16 hidden with
 *                 an fp32 gate is computed as hidden (hi + lo) with the gate
 *                 split into two bf16 parts (relative error of a product
 *                 <= 2^-16), so the result carries fp32-level accuracy.
 *   workspace     >= moe_workspace_size(p) bytes (partial logits of a split
 *                 over H when there are few tokens; unused otherwise).
 * Errors: MOE_ERR_INVALID (NULL), MOE_ERR_UNSUPPORTED (gate or act dtype),
 * MOE_ERR_WORKSPACE. */
int moe_router_gemm(const moe_params *p, const void *hidden, const void *gate_w,
                    int32_t gate_dtype, float *router_logits, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Router gate GEMM and top-k in one call (the gate, then select_experts),
 * with no fp32 [T, E] logits written unless asked for.
 * Passages: MoEGate (SGLang deepseek_v2 page: gate [n_routed_experts,
 * hidden_size], fp32 logits; a skinny GEMM at decode that the page gives
 * its own kernel) ahead of FusedMoE.select_experts (vLLM page) with the
 * DeepseekV2MoE grouped top-k arguments.
 *   hidden, gate_w, gate_dtype: as moe_router_gemm.
 *   e_score_correction_bias, topk_ids, topk_weights: as moe_topk.
 *   router_logits  [T, E] fp32 out, or NULL: the logits (bitwise those of
 *                  moe_router_gemm).
 * The GEMM writes partial logits of a split hidden dimension (decode sizes)
 * into the workspace and the top-k adds them in a fixed order as it reads
 * them, so the ids and weights are bitwise those of moe_router_gemm
 * followed by moe_topk.  With a bf16 hidden and at most 256 tokens this is
 * one launch: the router kernel's last blocks run the top-k once every
 * block's partial logits are written, counting arrivals in a device array
 * of the library (64 counters, taken in turn by successive calls, each left
 * at zero), so at most 64 such calls may be in flight on one device at a
 * time; otherwise a GEMM launch and a top-k launch.
 *   workspace      >= moe_workspace_size(p) bytes (unused when there is one
 *                  part and router_logits is given).  Calls in flight at the
 *                  same time need workspaces of their own.
 * Errors: as moe_router_gemm and moe_topk. */
int moe_router_topk(const moe_params *p, const void *hidden, const void *gate_w,
                    int32_t gate_dtype, const float *e_score_correction_bias,
                    int32_t *topk_ids, float *topk_weights, float *router_logits,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Router: top-k expert selection and routing weights per token.
 * Passage: FusedMoE.select_experts (vLLM page), grouped top-k and
 * e_score_correction_bias (vLLM page; DeepseekV2MoE TopK arguments and
 * MoEGate on the SGLang deepseek_v2 page).
 *   router_logits  [T, E] fp32.
 *   e_score_correction_bias  [E] fp32 or NULL (sigmoid scoring only; it moves
 *                  the selection, never the weights).
 *   topk_ids       [T, K] int32 out: selected experts in descending key
 *                  order; exact ties go to the lower expert index.
 *   topk_weights   [T, K] fp32 out: score of each selected expert (softmax
 *                  probability or sigmoid), divided by the K scores' sum if
 *                  renormalize, times routed_scaling_factor.
 * Selection key: the logit (softmax) or sigmoid(logit) + bias (sigmoid).
 * Grouped (G > 1): group j = experts [j*E/G, (j+1)*E/G); a group scores the
 * sum of its two largest keys with a bias, else its largest key; only the
 * TG best groups are eligible.
 * Errors: MOE_ERR_INVALID for K > E, E % G != 0, TG outside 1..G,
 * K > TG*E/G, a bias with softmax scoring, NULL pointers. */
int moe_topk(const moe_params *p, const float *router_logits,
             const float *e_score_correction_bias, int32_t *topk_ids,
             float *topk_weights, void *stream);

/* Expert-contiguous permutation of the T*K slots (slot i = t*K + k).
 * Passage: the dispatch step of FusedMoE.forward_impl (SGLang layer page:
 * dispatcher.dispatch -> run_moe_core -> dispatcher.combine).
 *   topk_ids       [T*K] int32, each in [0, E).
 *   expert_offsets [E+1] int32 out: expert e owns rows
 *                  [expert_offsets[e], expert_offsets[e+1]).
 *   sorted_slots   [T*K] int32 out: slot placed at each row; within an
 *                  expert, slots ascend (a stable sort, bit-exact).
 *   slot_to_row    [T*K] int32 out: inverse of sorted_slots.
 *   workspace      >= moe_workspace_size(p) bytes of device scratch.
 * Errors: MOE_ERR_INVALID (ids out of range are not detected on the
 * device: they are a precondition), MOE_ERR_WORKSPACE. */
int moe_align_permute(const moe_params *p, const int32_t *topk_ids,
                      int32_t *expert_offsets, int32_t *sorted_slots,
                      int32_t *slot_to_row, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Per-token-group-128 fp8 quantisation of the layer input, computed once and
 * fed to both the routed and the shared experts.
 * Passage: DeepseekV2MoE._maybe_quant_moe_input_once (SGLang deepseek_v2
 * page).
 *   hidden   [T, H] bf16.
 *   q        [T, H] e4m3 codes out;  scale  [T, H/128] fp32 out.
 * Errors: MOE_ERR_INVALID (H % 128, NULL), MOE_ERR_UNSUPPORTED (act dtype
 * not bf16). */
int moe_quant_act_fp8(const moe_params *p, const void *hidden, uint8_t *q,
                      float *scale, void *stream);

/* Rows of the shared expert.  With Is = m * I the shared expert's
 * intermediate dimension is taken as m consecutive slices of I (slice j:
 * gate rows [j*I, (j+1)*I) and up rows [Is + j*I, Is + (j+1)*I) of
 * shared_w13, columns [j*I, (j+1)*I) of shared_w2).  The down projection sums
 * over that dimension, so the shared MLP is the sum of the m slices' MLPs;
 * each slice is one more block of T rows of the grouped GEMMs: row
 * T*K + j*T + t holds token t through slice j.  Below, S = m when
 * num_shared_experts == 1, else 0. */

/* Gate/up grouped GEMM with SiLU-and-mul, row by row of the permutation.
 * Passage: FusedMoE w13 = [w1 (gate); w3 (up)] along the output dimension
 * (_load_w13, vLLM page), activation "silu" with is_act_and_mul;
 * DeepseekV2MLP gate_up_proj -> SiluAndMul (SGLang deepseek_v2 page).
 *   hidden       [T, H]: act dtype; for fp8 weights the e4m3 codes from
 *                moe_quant_act_fp8 with hidden_scale [T, H/128].
 *   w13          [E, 2I, H] packed by moe_pack_weights (+ w13_scale
 *                [E, 2I/128, H/128] row-major for fp8); [E, I, H] with
 *                non_gated.
 *   shared_w13   [2Is, H] ([Is, H] non-gated) packed (+ scale [2Is/128,
 *                H/128]) when num_shared_experts == 1, else NULL.
 *   expert_offsets, sorted_slots: from moe_align_permute.
 *   topk_weights [T, K] fp32 from moe_topk when router_weight_on_input
 *                (the w13 output of routed row r is scaled by its slot's
 *                weight before the activation, which equals scaling the
 *                input); else ignored and may be NULL.
 *   act          [T*K + T*S, I] out: row r < T*K holds silu(g) * u (or its
 *                variant, see moe_params) for the token of sorted_slots[r];
 *                rows T*K + j*T + t: token t through slice j of the shared
 *                expert.  bf16 for bf16 layers, fp32 for fp32 layers, e4m3
 *                codes for fp8 layers with act_scale [T*K + T*S, I/128] fp32
 *                out.
 * Errors: MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED (also weight_layout other
 * than MOE_LAYOUT_PACKED), MOE_ERR_WORKSPACE. */
int moe_grouped_gemm_w13_act(const moe_params *p, const void *hidden,
                             const float *hidden_scale, const void *w13,
                             const float *w13_scale, const void *shared_w13,
                             const float *shared_w13_scale,
                             const int32_t *expert_offsets,
                             const int32_t *sorted_slots,
                             const float *topk_weights, void *act,
                             float *act_scale, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Down grouped GEMM and the weighted combine back to token order.
 * Passage: FusedMoE w2 = down_proj (vLLM page), combine_output /
 * dispatcher.combine (both layer pages); DeepseekV2MoE adds the shared
 * expert with weight 1 and the routed part scaled by routed_scaling_factor
 * (already folded into topk_weights here).
 *   act, act_scale  from moe_grouped_gemm_w13_act.
 *   w2         [E, H, I] packed by moe_pack_weights (+ w2_scale
 *              [E, H/128, I/128] row-major for fp8).
 *   shared_w2  [H, Is] packed (+ scale [H/128, Is/128]) or NULL.
 *   topk_weights [T, K] fp32 from moe_topk; slot_to_row [T*K].
 *   out        [T, H] out_dtype:  out_t = sum_k w_{t,k} y_{row(t,k)}
 *              (+ sum_j y_{T*K+j*T+t} of the shared expert); with
 *              router_weight_on_input the rows are added unweighted (the
 *              weight went into the w13 call).  The sum over k runs in a
 *              fixed order in fp32, so results are bitwise reproducible.
 * Errors: MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED (also weight_layout other
 * than MOE_LAYOUT_PACKED), MOE_ERR_WORKSPACE. */
int moe_grouped_gemm_w2_combine(const moe_params *p, const void *act,
                                const float *act_scale, const void *w2,
                                const float *w2_scale, const void *shared_w2,
                                const float *shared_w2_scale,
                                const int32_t *expert_offsets,
                                const int32_t *sorted_slots,
                                const int32_t *slot_to_row,
                                const float *topk_weights, void *out,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* The whole layer: routing, permutation, (fp8: input quantisation),
 * w13 + SiLU-and-mul, w2 + weighted combine (+ shared expert).
 * Passage: FusedMoE.forward_native(hidden_states, router_logits) (vLLM
 * page); DeepseekV2MoE.forward_normal (SGLang deepseek_v2 page).
 *   hidden [T, H] act dtype; router_logits [T, E] fp32; weights as above.
 *   out [T, H] out_dtype.
 *   topk_ids_out [T, K] int32 / topk_weights_out [T, K] fp32: optional
 *   copies of the routing (NULL to skip).
 *   workspace >= moe_workspace_size(p) bytes.
 * Errors: as the calls it is made of (weight_layout must be
 * MOE_LAYOUT_PACKED). */
int moe_forward(const moe_params *p, const void *hidden,
                const float *router_logits,
                const float *e_score_correction_bias, const void *w13,
                const float *w13_scale, const void *w2, const float *w2_scale,
                const void *shared_w13, const float *shared_w13_scale,
                const void *shared_w2, const float *shared_w2_scale,
                void *out, int32_t *topk_ids_out, float *topk_weights_out,
                void *workspace, size_t workspace_bytes, void *stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same layer, arguments and result as moe_forward (bitwise), but no
 * workspace argument.  The workspace is a 64 MiB device array of the library
 * itself, one per GPU, held from the first call on that GPU until the process
 * ends.  Layers whose moe_workspace_size exceeds 64 MiB (decode and small
 * prefill batches fit: e.g. the DeepSeek-V3 shape up to a few hundred
 * tokens) return MOE_ERR_WORKSPACE before anything is launched; use
 * moe_forward with a workspace for those.  The call allocates nothing.  All
 * calls on one GPU share its array: calls that overlap in time on one GPU
 * (different streams, or host threads) race and give wrong results, so
 * serialise them (one stream).  `stream` must belong to the current device
 * (else MOE_ERR_INVALID).  Errors: as moe_forward, plus MOE_ERR_WORKSPACE
 * for layers beyond the array. */
int moe_forward_noalloc(const moe_params *p, const void *hidden,
                        const float *router_logits,
                        const float *e_score_correction_bias, const void *w13,
                        const float *w13_scale, const void *w2,
                        const float *w2_scale, const void *shared_w13,
                        const float *shared_w13_scale, const void *shared_w2,
                        const float *shared_w2_scale, void *out,
                        int32_t *topk_ids_out, float *topk_weights_out,
                        void *stream);

/* Measurement helpers (not steps of the method): what this GPU reaches, to
 * print beside the published peaks.  The caller times the launch.
 *   moe_peak_mfma_bf16: `blocks` blocks of 256 threads; every wave runs
 *     `iters` rounds of 8 independent 32x32x16 bf16 MFMAs (32768 FLOP each),
 *     i.e. blocks * 4 * iters * 8 * 32768 FLOP.  sink: blocks * 256 floats.
 *   moe_peak_read: `blocks` blocks of 256 threads read `bytes` (multiple of
 *     16, buffer 16-byte aligned) once with 16-byte loads, each block a
 *     contiguous share.  sink: blocks * 256 uint32.
 * Errors: MOE_ERR_INVALID for non-positive counts, NULL or misaligned
 * buffers; MOE_ERR_HIP. */
int moe_peak_mfma_bf16(int64_t iters, int32_t blocks, float *sink, void *stream);
int moe_peak_read(const void *buf, int64_t bytes, int32_t blocks, uint32_t *sink,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
