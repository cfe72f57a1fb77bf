"""Fused MoE layer object over the C ABI: holds the weights, owns one device
workspace and calls the library with torch's current stream.

Mirrors the argument surface of FusedMoE on the vLLM docs page
"vllm.model_executor.layers.fused_moe.layer" (num_experts, top_k,
hidden_size, intermediate_size, renormalize, num_expert_group, topk_group,
scoring_func, routed_scaling_factor, e_score_correction_bias) and its
forward(hidden_states, router_logits).  All compute happens in the HIP
library; this module allocates buffers and passes pointers.
"""
from __future__ import annotations

import torch

from . import binding as B

_DT = {"f32": B.F32, "bf16": B.BF16, "fp8": B.FP8_E4M3}
_TORCH_OUT = {B.F32: torch.float32, B.BF16: torch.bfloat16}


def params_for(cfg, T: int | None = None) -> B.MoeParams:
    """moe_params of a synth.MoEConfig."""
    T = cfg.T if T is None else T
    return B.make_params(
        num_tokens=T, num_experts=cfg.E, top_k=cfg.K, hidden_size=cfg.H,
        intermediate_size=cfg.I,
        scoring_func=B.SIGMOID if cfg.scoring == "sigmoid" else B.SOFTMAX,
        renormalize=cfg.renormalize, num_expert_group=cfg.n_group, topk_group=cfg.topk_group,
        routed_scaling_factor=cfg.rsf, act_dtype=_DT[cfg.act_dtype], weight_dtype=_DT[cfg.w_dtype],
        out_dtype=_DT[cfg.act_dtype], num_shared_experts=cfg.shared, non_gated=cfg.non_gated,
        swiglu_alpha=cfg.swiglu_alpha, swiglu_limit=cfg.swiglu_limit,
        router_weight_on_input=cfg.weight_on_input, weight_layout=B.LAYOUT_PACKED,
        shared_intermediate=cfg.shared_I if cfg.shared else 0)


_PACKED = ("w13", "w2", "shared_w13", "shared_w2")


class FusedMoE:
    """One layer: weights (w13, w2, optional scales and shared expert) plus a
    workspace sized for the largest token count seen so far.  The weight
    matrices are given row-major and kept in the library's packed layout
    (moe_pack_weights, done once here); scales stay as given."""

    def __init__(self, params: B.MoeParams, weights: dict):
        self.params = B.MoeParams.from_buffer_copy(params)
        self.params.weight_layout = B.LAYOUT_PACKED  # packed here, once
        self.w = {k: (B.pack_weights(v) if k in _PACKED and v is not None else v)
                  for k, v in weights.items()}
        self._ws = None

    def workspace(self, T: int) -> torch.Tensor:
        p = self._with_T(T)
        need = max(B.moe_workspace_size(p), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._ws

    def _with_T(self, T: int) -> B.MoeParams:
        p = B.MoeParams.from_buffer_copy(self.params)
        p.num_tokens = int(T)
        return p

    def forward(self, hidden, router_logits, e_score_correction_bias=None, out=None,
                topk_ids=None, topk_weights=None) -> torch.Tensor:
        T = hidden.shape[0]
        p = self._with_T(T)
        if out is None:
            out = torch.empty(T, p.hidden_size, dtype=_TORCH_OUT[p.out_dtype], device=hidden.device)
        ws = self.workspace(T)
        w = self.w
        B.moe_forward(p, hidden, router_logits, e_score_correction_bias, w["w13"],
                      w.get("w13_scale"), w["w2"], w.get("w2_scale"), w.get("shared_w13"),
                      w.get("shared_w13_scale"), w.get("shared_w2"), w.get("shared_w2_scale"),
                      out, topk_ids, topk_weights, ws)
        return out

    __call__ = forward


class Stages:
    """Buffers for running the layer as its separate entry points
    (moe_topk -> moe_align_permute -> [moe_quant_act_fp8] ->
    moe_grouped_gemm_w13_act -> moe_grouped_gemm_w2_combine)."""

    def __init__(self, layer: FusedMoE, T: int):
        p = layer._with_T(T)
        self.p = p
        self.layer = layer
        dev = "cuda"
        E, K, H, I = p.num_experts, p.top_k, p.hidden_size, p.intermediate_size
        # rows of the shared expert: T per I-wide slice of its intermediate size
        slices = (p.shared_intermediate // I if p.shared_intermediate else 1) if p.num_shared_experts else 0
        R = T * K + T * slices
        fp8 = p.weight_dtype == B.FP8_E4M3
        self.ids = torch.empty(T, K, dtype=torch.int32, device=dev)
        self.weights = torch.empty(T, K, dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.sorted = torch.empty(T * K, dtype=torch.int32, device=dev)
        self.inv = torch.empty(T * K, dtype=torch.int32, device=dev)
        if fp8:
            self.xq = torch.empty(T, H, dtype=torch.uint8, device=dev)
            self.xs = torch.empty(T, H // 128, dtype=torch.float32, device=dev)
            self.act = torch.empty(R, I, dtype=torch.uint8, device=dev)
            self.act_scale = torch.empty(R, I // 128, dtype=torch.float32, device=dev)
        else:
            self.xq = self.xs = self.act_scale = None
            self.act = torch.empty(R, I, dtype=_TORCH_OUT[p.act_dtype], device=dev)
        self.out = torch.empty(T, H, dtype=_TORCH_OUT[p.out_dtype], device=dev)
        self.ws = layer.workspace(T)

    def topk(self, router_logits, bias=None):
        B.moe_topk(self.p, router_logits, bias, self.ids, self.weights)

    def align(self):
        B.moe_align_permute(self.p, self.ids, self.offsets, self.sorted, self.inv, self.ws)

    def quant(self, hidden):
        B.moe_quant_act_fp8(self.p, hidden, self.xq, self.xs)

    def w13(self, hidden):
        w = self.layer.w
        fp8 = self.xq is not None
        B.moe_grouped_gemm_w13_act(self.p, self.xq if fp8 else hidden, self.xs, w["w13"],
                                   w.get("w13_scale"), w.get("shared_w13"),
                                   w.get("shared_w13_scale"), self.offsets, self.sorted,
                                   self.weights, self.act, self.act_scale, self.ws)

    def w2(self):
        w = self.layer.w
        B.moe_grouped_gemm_w2_combine(self.p, self.act, self.act_scale, w["w2"], w.get("w2_scale"),
                                      w.get("shared_w2"), w.get("shared_w2_scale"), self.offsets,
                                      self.sorted, self.inv, self.weights, self.out, self.ws)

    def run(self, hidden, router_logits, bias=None):
        self.topk(router_logits, bias)
        self.align()
        if self.xq is not None:
            self.quant(hidden)
        self.w13(hidden)
        self.w2()
        return self.out
