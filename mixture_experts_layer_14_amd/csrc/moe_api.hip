// moe_api.hip -- the C ABI (include/moe.h): host-side validation, workspace
// layout and kernel launches.  Nothing here synchronises with the device or
// allocates memory.
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;
constexpr int kMaxSharedSlices = 16;  // shared_intermediate <= 16 * I

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool fp8_layer(const moe_params* p) { return p->weight_dtype == MOE_DTYPE_FP8_E4M3; }

size_t act_elt(const moe_params* p) {
    if (fp8_layer(p)) return 1;
    return p->act_dtype == MOE_DTYPE_F32 ? 4 : 2;
}

int64_t routed_rows(const moe_params* p) { return p->num_tokens * p->top_k; }
// I-wide slices of the shared expert (its intermediate size over I)
int shared_slices(const moe_params* p) {
    if (!p->num_shared_experts) return 0;
    return p->shared_intermediate > 0 ? p->shared_intermediate / p->intermediate_size : 1;
}
int64_t all_rows(const moe_params* p) { return routed_rows(p) + shared_slices(p) * p->num_tokens; }

// Shape/parameter checks shared by every call.
int check_params(const moe_params* p) {
    if (!p) return MOE_ERR_INVALID;
    if (p->num_tokens < 0 || p->num_experts < 1 || p->num_experts > kMaxExperts) return MOE_ERR_INVALID;
    if (p->top_k < 1 || p->top_k > p->num_experts) return MOE_ERR_INVALID;
    if (p->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (p->hidden_size <= 0 || p->intermediate_size <= 0) return MOE_ERR_INVALID;
    if (p->scoring_func != MOE_SCORING_SOFTMAX && p->scoring_func != MOE_SCORING_SIGMOID)
        return MOE_ERR_INVALID;
    if (p->num_shared_experts < 0) return MOE_ERR_INVALID;
    if (p->num_shared_experts > 1) return MOE_ERR_UNSUPPORTED;
    if (p->weight_layout != MOE_LAYOUT_ROW_MAJOR && p->weight_layout != MOE_LAYOUT_PACKED)
        return MOE_ERR_INVALID;
    if (p->shared_intermediate < 0) return MOE_ERR_INVALID;
    if (p->shared_intermediate > 0) {
        if (!p->num_shared_experts) return MOE_ERR_INVALID;
        // the pages' shared expert is n_shared_experts routed-sized MLPs wide
        if (p->shared_intermediate % p->intermediate_size) return MOE_ERR_UNSUPPORTED;
        if (p->shared_intermediate / p->intermediate_size > kMaxSharedSlices) return MOE_ERR_UNSUPPORTED;
    }
    const int G = p->num_expert_group;
    if (G < 0) return MOE_ERR_INVALID;
    if (G > 1) {
        if (p->num_experts % G != 0) return MOE_ERR_INVALID;
        if (p->topk_group < 1 || p->topk_group > G) return MOE_ERR_INVALID;
        if (p->top_k > p->topk_group * (p->num_experts / G)) return MOE_ERR_INVALID;
        if (G > kMaxGroups) return MOE_ERR_UNSUPPORTED;
    }
    const int a = p->act_dtype, w = p->weight_dtype, o = p->out_dtype;
    const bool ok = (a == MOE_DTYPE_F32 && w == MOE_DTYPE_F32 && o == MOE_DTYPE_F32) ||
                    (a == MOE_DTYPE_BF16 && w == MOE_DTYPE_BF16 && o == MOE_DTYPE_BF16) ||
                    (a == MOE_DTYPE_BF16 && w == MOE_DTYPE_FP8_E4M3 && o == MOE_DTYPE_BF16);
    if (a < 0 || a > 2 || w < 0 || w > 2 || o < 0 || o > 2) return MOE_ERR_INVALID;
    if (!ok) return MOE_ERR_UNSUPPORTED;
    const int mult = fp8_layer(p) ? 128 : 64;
    if (p->hidden_size % mult || p->intermediate_size % mult) return MOE_ERR_INVALID;
    // activation variants: a clamp needs the gated form; the fp8 paths run
    // the gated SiLU family only and quantise x itself (no input weighting)
    if (p->non_gated != 0 && p->non_gated != 1) return MOE_ERR_INVALID;
    if (p->router_weight_on_input != 0 && p->router_weight_on_input != 1) return MOE_ERR_INVALID;
    if (!(p->swiglu_alpha >= 0.0f) || !(p->swiglu_limit >= 0.0f)) return MOE_ERR_INVALID;  // NaN too
    if (p->non_gated && p->swiglu_limit > 0.0f) return MOE_ERR_INVALID;
    if (fp8_layer(p) && (p->non_gated || p->router_weight_on_input)) return MOE_ERR_UNSUPPORTED;
    // rows and element offsets held in int32 on the device
    if (all_rows(p) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe::GroupedProblem problem(const moe_params* p, moe::TileTableKey* built = nullptr) {
    moe::GroupedProblem g;
    g.built = built;
    g.dtype = p->weight_dtype;
    g.T = p->num_tokens;
    g.K = p->top_k;
    g.E = p->num_experts;
    g.shared = shared_slices(p);
    g.H = p->hidden_size;
    g.I = p->intermediate_size;
    g.Is = g.shared * g.I;
    g.gated = p->non_gated ? 0 : 1;
    g.alpha = p->swiglu_alpha > 0.0f ? p->swiglu_alpha : 1.0f;
    g.limit = p->swiglu_limit;
    g.weight_in = p->router_weight_on_input;
    return g;
}

size_t w13_scratch(const moe_params* p) { return moe::gemm_tile_workspace_bytes(problem(p)); }
size_t w2_scratch(const moe_params* p) {
    const moe::GroupedProblem g = problem(p);
    return moe::gemm_tile_workspace_bytes(g) + moe::w2_rows_workspace_bytes(g);
}
size_t align_scratch(const moe_params* p) {
    return align256(moe::align_workspace_bytes(routed_rows(p), p->num_experts));
}

// Workspace of moe_forward: routing, permutation, quantised input,
// activations, then a scratch region reused by each stage.
struct ForwardLayout {
    size_t ids, weights, offsets, sorted, inv, xq, xs, act, act_scale, scratch, total;
};

ForwardLayout forward_layout(const moe_params* p) {
    ForwardLayout L{};
    const size_t TK = static_cast<size_t>(routed_rows(p));
    const size_t T = static_cast<size_t>(p->num_tokens);
    const size_t H = p->hidden_size, I = p->intermediate_size;
    const size_t R = static_cast<size_t>(all_rows(p));
    size_t off = 0;
    L.ids = off; off += align256(TK * 4);
    L.weights = off; off += align256(TK * 4);
    L.offsets = off; off += align256((p->num_experts + 1) * 4);
    L.sorted = off; off += align256(TK * 4);
    L.inv = off; off += align256(TK * 4);
    L.xq = off; off += fp8_layer(p) ? align256(T * H) : 0;
    L.xs = off; off += fp8_layer(p) ? align256(T * (H / 128) * 4) : 0;
    // rows rounded up to 16: moe_forward may keep act in the packed layout
    L.act = off; off += align256((R + 15) / 16 * 16 * I * act_elt(p));
    L.act_scale = off; off += fp8_layer(p) ? align256(R * (I / 128) * 4) : 0;
    L.scratch = off;
    size_t s = align_scratch(p);
    if (w13_scratch(p) > s) s = w13_scratch(p);
    if (w2_scratch(p) > s) s = w2_scratch(p);
    // covers moe_router_gemm's partial logits too (a call of its own)
    const size_t r = moe::router_workspace_bytes(p->num_tokens, p->num_experts, p->hidden_size,
                                                 p->act_dtype);
    if (off + s < r) s = r - off;
    L.total = off + s;
    return L;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
    return MOE_ERR_HIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int check_topk_args(const moe_params* p, const float* logits, const float* bias, const int32_t* ids,
                    const float* w) {
    if (!logits || !ids || !w) return MOE_ERR_INVALID;
    if (bias && p->scoring_func != MOE_SCORING_SIGMOID) return MOE_ERR_INVALID;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t moe_workspace_size(const moe_params* p) {
    if (check_params(p) != MOE_OK) return 0;
    return forward_layout(p).total;
}

int moe_topk(const moe_params* p, const float* router_logits, const float* e_score_correction_bias,
             int32_t* topk_ids, float* topk_weights, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    st = check_topk_args(p, router_logits, e_score_correction_bias, topk_ids, topk_weights);
    if (st != MOE_OK) return st;
    const int G = p->num_expert_group > 1 ? p->num_expert_group : 1;
    return hip_status(moe::launch_topk(router_logits, 1, nullptr, e_score_correction_bias, p->num_tokens,
                                       p->num_experts, p->top_k, p->scoring_func,
                                       p->renormalize ? 1 : 0, G, G > 1 ? p->topk_group : 1,
                                       p->routed_scaling_factor, topk_ids, topk_weights,
                                       as_stream(stream)));
}

int moe_align_permute(const moe_params* p, const int32_t* topk_ids, int32_t* expert_offsets,
                      int32_t* sorted_slots, int32_t* slot_to_row, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!topk_ids || !expert_offsets || !sorted_slots || !slot_to_row) return MOE_ERR_INVALID;
    if (!workspace || workspace_bytes < align_scratch(p)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_align(topk_ids, routed_rows(p), p->num_experts, expert_offsets,
                                        sorted_slots, slot_to_row, workspace, as_stream(stream)));
}

int moe_pack_weights(const void* src, void* dst, int64_t matrices, int64_t rows,
                     int64_t row_bytes, void* stream) {
    if (matrices < 0 || rows < 0 || row_bytes < 0) return MOE_ERR_INVALID;
    if (rows % 16 != 0 || row_bytes % 64 != 0) return MOE_ERR_INVALID;
    if (matrices == 0 || rows == 0 || row_bytes == 0) return MOE_OK;
    if (!src || !dst) return MOE_ERR_INVALID;
    // the product must fit the address space; then reject any overlap
    if (rows > INT64_MAX / row_bytes || matrices > INT64_MAX / (rows * row_bytes)) return MOE_ERR_INVALID;
    const uint64_t n = static_cast<uint64_t>(matrices * rows * row_bytes);
    const uint64_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + n && d0 < s0 + n) return MOE_ERR_INVALID;
    if ((s0 | d0) & 15) return MOE_ERR_INVALID;
    return hip_status(moe::launch_pack_weights(src, dst, matrices, rows, row_bytes, as_stream(stream)));
}

int moe_quant_act_fp8(const moe_params* p, const void* hidden, uint8_t* q, float* scale,
                      void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!hidden || !q || !scale) return MOE_ERR_INVALID;
    if (p->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->hidden_size % 128) return MOE_ERR_INVALID;
    return hip_status(moe::launch_quant_fp8(hidden, p->num_tokens, p->hidden_size, q, scale,
                                            as_stream(stream)));
}

}  // extern "C"

namespace {

// The two GEMM entry points; `built` (moe_forward only) records the tile
// table in the workspace across them, and marks the act buffer as
// moe_forward's own (its layout is then the kernels' choice).
int w13_act(const moe_params* p, const void* hidden, const float* hidden_scale, const void* w13,
            const float* w13_scale, const void* shared_w13, const float* shared_w13_scale,
            const int32_t* expert_offsets, const int32_t* sorted_slots, const float* topk_weights,
            void* act, float* act_scale, void* workspace, size_t workspace_bytes, void* stream,
            moe::TileTableKey* built) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->weight_layout != MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!hidden || !w13 || !expert_offsets || !sorted_slots || !act) return MOE_ERR_INVALID;
    if (p->num_shared_experts && !shared_w13) return MOE_ERR_INVALID;
    if (p->router_weight_on_input && !topk_weights) return MOE_ERR_INVALID;
    if (fp8_layer(p) && (!hidden_scale || !w13_scale || !act_scale ||
                         (p->num_shared_experts && !shared_w13_scale)))
        return MOE_ERR_INVALID;
    if (!workspace || workspace_bytes < w13_scratch(p)) return MOE_ERR_WORKSPACE;
    moe::GroupedProblem g = problem(p, built);
    g.act_packed = built && moe::act_packed_ok(g);  // moe_forward's own act buffer
    return hip_status(moe::launch_w13(g, hidden, hidden_scale, w13, w13_scale, shared_w13,
                                      shared_w13_scale, expert_offsets, sorted_slots,
                                      topk_weights, act, act_scale, workspace,
                                      as_stream(stream)));
}

int w2_combine(const moe_params* p, const void* act, const float* act_scale, const void* w2,
               const float* w2_scale, const void* shared_w2, const float* shared_w2_scale,
               const int32_t* expert_offsets, const int32_t* sorted_slots,
               const int32_t* slot_to_row, const float* topk_weights, void* out, void* workspace,
               size_t workspace_bytes, void* stream, moe::TileTableKey* built) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->weight_layout != MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!act || !w2 || !expert_offsets || !sorted_slots || !slot_to_row || !topk_weights || !out)
        return MOE_ERR_INVALID;
    if (p->num_shared_experts && !shared_w2) return MOE_ERR_INVALID;
    if (fp8_layer(p) && (!act_scale || !w2_scale || (p->num_shared_experts && !shared_w2_scale)))
        return MOE_ERR_INVALID;
    if (!workspace || workspace_bytes < w2_scratch(p)) return MOE_ERR_WORKSPACE;
    moe::GroupedProblem g = problem(p, built);
    g.act_packed = built && moe::act_packed_ok(g);  // moe_forward's own act buffer
    return hip_status(moe::launch_w2_combine(g, act, act_scale, w2, w2_scale, shared_w2,
                                             shared_w2_scale, expert_offsets, sorted_slots,
                                             slot_to_row, topk_weights, out, workspace,
                                             as_stream(stream)));
}

}  // namespace

extern "C" {

int moe_grouped_gemm_w13_act(const moe_params* p, const void* hidden, const float* hidden_scale,
                             const void* w13, const float* w13_scale, const void* shared_w13,
                             const float* shared_w13_scale, const int32_t* expert_offsets,
                             const int32_t* sorted_slots, const float* topk_weights, void* act,
                             float* act_scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return w13_act(p, hidden, hidden_scale, w13, w13_scale, shared_w13, shared_w13_scale,
                   expert_offsets, sorted_slots, topk_weights, act, act_scale, workspace,
                   workspace_bytes, stream, nullptr);
}

int moe_grouped_gemm_w2_combine(const moe_params* p, const void* act, const float* act_scale,
                                const void* w2, const float* w2_scale, const void* shared_w2,
                                const float* shared_w2_scale, const int32_t* expert_offsets,
                                const int32_t* sorted_slots, const int32_t* slot_to_row,
                                const float* topk_weights, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return w2_combine(p, act, act_scale, w2, w2_scale, shared_w2, shared_w2_scale, expert_offsets,
                      sorted_slots, slot_to_row, topk_weights, out, workspace, workspace_bytes,
                      stream, nullptr);
}

int moe_router_gemm(const moe_params* p, const void* hidden, const void* gate_w,
                    int32_t gate_dtype, float* router_logits, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (gate_dtype != MOE_DTYPE_F32 && gate_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!hidden || !gate_w || !router_logits) return MOE_ERR_INVALID;
    if (p->act_dtype != MOE_DTYPE_F32 && p->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    // partial logits of a split H only
    const int parts = p->act_dtype == MOE_DTYPE_BF16
                          ? moe::router_parts(p->num_tokens, p->num_experts, p->hidden_size) : 1;
    const size_t need = parts > 1 ? static_cast<size_t>(parts) * p->num_tokens * p->num_experts * 4 : 0;
    if (need && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_router(hidden, p->act_dtype, gate_w, gate_dtype, p->num_tokens,
                                         p->num_experts, p->hidden_size, router_logits, workspace,
                                         as_stream(stream)));
}

int moe_router_topk(const moe_params* p, const void* hidden, const void* gate_w, int32_t gate_dtype,
                    const float* e_score_correction_bias, int32_t* topk_ids, float* topk_weights,
                    float* router_logits, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (gate_dtype != MOE_DTYPE_F32 && gate_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!hidden || !gate_w || !topk_ids || !topk_weights) return MOE_ERR_INVALID;
    if (e_score_correction_bias && p->scoring_func != MOE_SCORING_SIGMOID) return MOE_ERR_INVALID;
    if (p->act_dtype != MOE_DTYPE_F32 && p->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    const int64_t T = p->num_tokens;
    const int E = p->num_experts, H = p->hidden_size;
    const int parts = p->act_dtype == MOE_DTYPE_BF16 ? moe::router_parts(T, E, H) : 1;
    // one part straight into the caller's logits when it keeps them
    const bool direct = parts == 1 && router_logits;
    const size_t need = direct ? 0 : static_cast<size_t>(parts) * T * E * 4;
    if (need && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    float* partials = direct ? router_logits : static_cast<float*>(workspace);
    const int G = p->num_expert_group > 1 ? p->num_expert_group : 1;
    if (moe::router_topk_one_launch(T, E, H, p->act_dtype))
        return hip_status(moe::launch_router_topk(hidden, gate_w, gate_dtype, T, E, H, partials,
                                                  direct ? nullptr : router_logits, e_score_correction_bias,
                                                  p->top_k, p->scoring_func, p->renormalize ? 1 : 0, G,
                                                  G > 1 ? p->topk_group : 1, p->routed_scaling_factor,
                                                  topk_ids, topk_weights, as_stream(stream)));
    int got = 1;
    hipError_t err = moe::launch_router_partials(hidden, p->act_dtype, gate_w, gate_dtype, T, E, H,
                                                 partials, &got, as_stream(stream));
    if (err != hipSuccess) return hip_status(err);
    return hip_status(moe::launch_topk(partials, got, direct ? nullptr : router_logits,
                                       e_score_correction_bias, T, E, p->top_k, p->scoring_func,
                                       p->renormalize ? 1 : 0, G, G > 1 ? p->topk_group : 1,
                                       p->routed_scaling_factor, topk_ids, topk_weights,
                                       as_stream(stream)));
}

int moe_forward(const moe_params* p, const void* hidden, const float* router_logits,
                const float* e_score_correction_bias, const void* w13, const float* w13_scale,
                const void* w2, const float* w2_scale, const void* shared_w13,
                const float* shared_w13_scale, const void* shared_w2,
                const float* shared_w2_scale, void* out, int32_t* topk_ids_out,
                float* topk_weights_out, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    if (p->weight_layout != MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0) return MOE_OK;  // empty batch: nothing to do
    if (!hidden || !router_logits || !w13 || !w2 || !out) return MOE_ERR_INVALID;
    if (e_score_correction_bias && p->scoring_func != MOE_SCORING_SIGMOID) return MOE_ERR_INVALID;
    if (p->num_shared_experts && (!shared_w13 || !shared_w2)) return MOE_ERR_INVALID;
    if (fp8_layer(p) && (!w13_scale || !w2_scale ||
                         (p->num_shared_experts && (!shared_w13_scale || !shared_w2_scale))))
        return MOE_ERR_INVALID;
    const ForwardLayout L = forward_layout(p);
    if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
    float* wts = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(ws + L.weights);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
    void* scratch = ws + L.scratch;
    const size_t scratch_bytes = L.total - L.scratch;

    st = moe_topk(p, router_logits, e_score_correction_bias, ids, wts, stream);
    if (st != MOE_OK) return st;
    st = moe_align_permute(p, ids, offsets, sorted, inv, scratch, scratch_bytes, stream);
    if (st != MOE_OK) return st;
    const void* a1 = hidden;
    const float* a1_scale = nullptr;
    if (fp8_layer(p)) {
        uint8_t* xq = ws + L.xq;
        float* xs = reinterpret_cast<float*>(ws + L.xs);
        st = moe_quant_act_fp8(p, hidden, xq, xs, stream);
        if (st != MOE_OK) return st;
        a1 = xq;
        a1_scale = xs;
    }
    void* act = ws + L.act;
    float* act_scale = fp8_layer(p) ? reinterpret_cast<float*>(ws + L.act_scale) : nullptr;
    // both GEMMs use the same scratch region, so w2 reuses w13's tile table
    // when it would build the same one
    moe::TileTableKey built;
    st = w13_act(p, a1, a1_scale, w13, w13_scale, shared_w13, shared_w13_scale, offsets, sorted,
                 wts, act, act_scale, scratch, scratch_bytes, stream, &built);
    if (st != MOE_OK) return st;
    return w2_combine(p, act, act_scale, w2, w2_scale, shared_w2, shared_w2_scale, offsets,
                      sorted, inv, wts, out, scratch, scratch_bytes, stream, &built);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// moe_forward_noalloc: moe_forward on a workspace of the library's own, for
// callers that cannot allocate device memory.
// ---------------------------------------------------------------------------

// The workspace of moe_forward_noalloc: a device array of the library, one
// copy on each GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is handed to kernels.
static constexpr size_t kNoAllocBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
int scratch_address(void* stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kNoAllocMaxDevices) return MOE_ERR_UNSUPPORTED;
    if (stream) {  // the stream must belong to the current device
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return MOE_ERR_HIP;
        if (sdev != dev) return MOE_ERR_INVALID;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_params* p, const void* hidden, const float* router_logits,
                        const float* e_score_correction_bias, const void* w13,
                        const float* w13_scale, const void* w2, const float* w2_scale,
                        const void* shared_w13, const float* shared_w13_scale,
                        const void* shared_w2, const float* shared_w2_scale, void* out,
                        int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
    int st = check_params(p);
    if (st != MOE_OK) return st;
    // larger layers than the array holds take moe_forward with a workspace
    if (forward_layout(p).total > kNoAllocBytes) return MOE_ERR_WORKSPACE;
    if (p->num_tokens == 0) return moe_forward(p, hidden, router_logits, e_score_correction_bias, w13,
                                               w13_scale, w2, w2_scale, shared_w13, shared_w13_scale,
                                               shared_w2, shared_w2_scale, out, topk_ids_out,
                                               topk_weights_out, nullptr, 0, stream);
    void* ws = nullptr;
    st = scratch_address(stream, &ws);
    if (st != MOE_OK) return st;
    // every kernel of moe_forward writes the workspace regions it reads
    // later in the same call, so nothing has to start at zero
    return moe_forward(p, hidden, router_logits, e_score_correction_bias, w13, w13_scale, w2,
                       w2_scale, shared_w13, shared_w13_scale, shared_w2, shared_w2_scale, out,
                       topk_ids_out, topk_weights_out, ws, kNoAllocBytes, stream);
}

}  // extern "C"
