"""Helpers of the GPU parity tests: hand the very bytes the GPU saw to the
CPU oracle, and compare to the stated bars."""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_layer_14_amd import synth
from oracle import oracle as O

# Output bars: max|err| / max|ref| over the compared rows (fp32 accumulation).
TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8": 6e-2}
# Routing weights are fp32 on the GPU, fp64 in the oracle.
WEIGHT_RTOL = 2e-6


def oracle_dtype(cfg):
    return {"f32": O.F32, "bf16": O.BF16, "fp8": O.E4M3}[cfg.w_dtype]


def to_host_bits(t):
    return synth.tensor_bits(t)


def oracle_layer(cfg, inp: dict, T: int, experts=None) -> dict:
    """Oracle arrays from the device inputs; `experts` limits which experts'
    weights are copied to the host (None = all)."""
    E = cfg.E
    need = range(E) if experts is None else sorted(set(int(e) for e in experts))

    def per_expert(key):
        t = inp.get(key)
        if t is None:
            return None
        return {e: to_host_bits(t[e]) for e in need}

    L = dict(T=T, E=E, K=cfg.K, H=cfg.H, I=cfg.I,
             scoring=O.SIGMOID if cfg.scoring == "sigmoid" else O.SOFTMAX,
             renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
             routed_scaling_factor=cfg.rsf,
             x_dtype=O.F32 if cfg.act_dtype == "f32" else O.BF16,
             w_dtype=oracle_dtype(cfg), act_fp8=cfg.fp8,
             hidden=to_host_bits(inp["hidden"]),
             logits=to_host_bits(inp["router_logits"]),
             bias=to_host_bits(inp.get("e_score_correction_bias")),
             w13=per_expert("w13"), w2=per_expert("w2"),
             w13_scale=per_expert("w13_scale"), w2_scale=per_expert("w2_scale"),
             gated=not cfg.non_gated,
             act_alpha=cfg.swiglu_alpha if cfg.swiglu_alpha > 0 else 1.0,
             clamp_limit=cfg.swiglu_limit, weight_on_input=cfg.weight_on_input,
             shared_I=cfg.shared_I if cfg.shared else 0)
    if cfg.shared:
        L["shared_w13"] = to_host_bits(inp["shared_w13"])
        L["shared_w2"] = to_host_bits(inp["shared_w2"])
        L["shared_w13_scale"] = to_host_bits(inp.get("shared_w13_scale"))
        L["shared_w2_scale"] = to_host_bits(inp.get("shared_w2_scale"))
    return L


def oracle_route(cfg, logits_np, bias_np):
    return O.route(logits_np, cfg.K, bias=bias_np,
                   scoring=O.SIGMOID if cfg.scoring == "sigmoid" else O.SOFTMAX,
                   renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
                   routed_scaling_factor=cfg.rsf)


def last_row_tokens(offsets: np.ndarray, sorted_slots: np.ndarray, K: int, most: int = 64) -> list:
    """Tokens of the last permuted row of each non-empty expert segment (the
    rows of each expert's ragged or tail m-tile), thinned to at most `most`
    experts taken evenly across the non-empty ones."""
    E = offsets.size - 1
    ends = [int(offsets[e + 1]) - 1 for e in range(E) if offsets[e + 1] > offsets[e]]
    if len(ends) > most:
        ends = [ends[i] for i in np.linspace(0, len(ends) - 1, most).round().astype(int)]
    return (sorted_slots[ends] // K).tolist()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
