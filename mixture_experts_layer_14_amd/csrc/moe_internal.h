// moe_internal.h -- host-side interface between the kernel translation units
// and the C ABI layer (not installed; the public interface is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One m-tile of the grouped GEMMs: rows [row0, row1) of the permuted order,
// all owned by `expert` (expert == E + j denotes slice j of the shared
// expert).
struct Tile {
    int32_t expert;
    int32_t row0;
    int32_t row1;
    int32_t group;  // (index of the group's first m-tile) * 256 + m-tiles in the group
};

// A group of one expert's m-tiles in a schedule with tail tiles: cnt main
// m-tiles from first_tile on, then (tail = 1) one tail m-tile; the group's
// block positions start at unit first_unit.
struct GroupUnit {
    int32_t first_tile;
    int32_t cnt;
    int32_t tail;
    int32_t first_unit;
};

// Top-k routing of `parts` partial logit arrays [parts][T][E] (summed in
// part order; 1: plain logits), optionally storing the summed logits.
hipError_t launch_topk(const float* logits, int parts, float* logits_out, const float* bias,
                       int64_t T, int E, int K, int scoring, int renorm, int G, int TG, float rsf,
                       int32_t* ids, float* weights, hipStream_t stream);

int64_t align_chunk(int64_t n);
size_t align_workspace_bytes(int64_t n, int E);
hipError_t launch_align(const int32_t* ids, int64_t n, int E, int32_t* offsets,
                        int32_t* sorted_slots, int32_t* slot_to_row, void* ws,
                        hipStream_t stream);

// Grouped GEMM problem shared by the two expert GEMMs.
// What the tile table at the start of a GEMM workspace was last built for.
// moe_forward hands one record to both of its GEMM calls, so the second skips
// a build identical to the first (same workspace, offsets and tile plan).
struct TileTableKey {
    const void* ws = nullptr;
    const int32_t* offsets = nullptr;
    int bm = 0, tail_rows = 0, split_nn = 0, ext_rows = 0;
};

struct GroupedProblem {
    int dtype;             // MOE_DTYPE_* of A and B (F32, BF16, FP8_E4M3)
    int64_t T;             // tokens
    int K;                 // top_k
    int E;                 // routed experts
    int shared;            // slices of the shared expert (0 = none), each I
                           // wide: slice j owns rows T*K + j*T .. T*K + j*T + T-1
    int H, I;              // hidden, intermediate
    int Is;                // intermediate size of the shared expert (shared * I)
    // activation variants (moe_params): gated SiLU-and-mul (1) or SiLU of
    // one projection (0); SiLU slope; clamp limit (0: none); routing weight
    // applied to the expert input instead of its output
    int gated = 1;
    float alpha = 1.0f;
    float limit = 0.0f;
    int weight_in = 0;
    // act between the two GEMMs in the weights' packed layout (moe_forward's
    // own buffer, rows rounded up to 16; shapes act_packed_ok accepts)
    bool act_packed = false;
    // record of the table in the workspace (null: always build)
    TileTableKey* built = nullptr;
};

// Whether both GEMMs of the problem run tile kernels, which can hand the act
// over in the packed layout.
bool act_packed_ok(const GroupedProblem& p);

// Scratch bytes of one grouped GEMM launch (tile table).
size_t gemm_tile_workspace_bytes(const GroupedProblem& p);
// Scratch bytes of the w2 GEMM's per-row outputs before the combine.
size_t w2_rows_workspace_bytes(const GroupedProblem& p);

// Packed weight layout (see moe_pack_weights): matrices x rows x row_bytes.
hipError_t launch_pack_weights(const void* src, void* dst, int64_t matrices, int64_t rows,
                               int64_t row_bytes, hipStream_t stream);

hipError_t launch_w13(const GroupedProblem& p, const void* hidden, const float* hidden_scale,
                      const void* w13, const float* w13_scale, const void* shared_w13,
                      const float* shared_w13_scale, const int32_t* offsets,
                      const int32_t* sorted_slots, const float* topk_weights, void* act,
                      float* act_scale, void* ws, hipStream_t stream);

hipError_t launch_w2_combine(const GroupedProblem& p, const void* act, const float* act_scale,
                             const void* w2, const float* w2_scale, const void* shared_w2,
                             const float* shared_w2_scale, const int32_t* offsets,
                             const int32_t* sorted_slots, const int32_t* slot_to_row,
                             const float* topk_weights, void* out, void* ws,
                             hipStream_t stream);

// Router gate logits (moe_router.hip); dtypes are MOE_DTYPE_* values.
// Parts of H the bf16 GEMM splits into (partial logits summed by the consumer).
int router_parts(int64_t T, int E, int H);
// Workspace of the fused router + top-k: the partial logits, or one logits
// array when there is one part (the larger of the two router uses).
size_t router_workspace_bytes(int64_t T, int E, int H, int act_dtype);
// Partial logits [parts][T][E] into `partials`; *parts_out = parts used.
hipError_t launch_router_partials(const void* hidden, int act_dtype, const void* gate,
                                  int gate_dtype, int64_t T, int E, int H, float* partials,
                                  int* parts_out, hipStream_t stream);
// Logits [T, E] (partials, when H is split, in ws, then summed).
// Router gate GEMM and top-k in one launch (bf16 hidden, few tokens: the
// shapes router_topk_one_launch accepts); partials as for
// launch_router_partials.  Overlapping such launches on one device race.
bool router_topk_one_launch(int64_t T, int E, int H, int act_dtype);
hipError_t launch_router_topk(const void* hidden, const void* gate, int gate_dtype, int64_t T, int E,
                              int H, float* partials, float* logits_out, const float* bias, int K,
                              int scoring, int renorm, int G, int TG, float rsf, int32_t* ids,
                              float* weights, hipStream_t stream);
hipError_t launch_router(const void* hidden, int act_dtype, const void* gate, int gate_dtype,
                         int64_t T, int E, int H, float* logits, void* ws, hipStream_t stream);

hipError_t launch_quant_fp8(const void* hidden, int64_t T, int H, uint8_t* q, float* scale,
                            hipStream_t stream);

}  // namespace moe
