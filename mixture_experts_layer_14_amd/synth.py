"""Seeded synthetic inputs for the fused MoE layer forward.

Used by the tests and by bench.py.  This module draws inputs only; it holds
none of the layer's arithmetic and is imported neither by the HIP binding nor
by the CPU oracle.  Both sides receive the very same bytes from it.

Recipe (shapes and distributions of the workloads the pages describe: a
Mixtral-shape layer, a many-expert Qwen-style layer, and the DeepSeek-V3
MoE block of the SGLang page "srt/models/deepseek_v2.py"):

* hidden ~ N(0, 1), rounded to the activation dtype (bf16 by round-to-nearest-
  even);
* expert weights ~ N(0, w_std) drawn in fp32, then rounded to bf16, or block-
  quantised to OCP e4m3 with one fp32 scale per 128 x 128 block
  (scale = amax / 448, codes = e4m3(w / scale));
* router logits ~ N(0, 1) in fp32, plus a per-expert skew
  b_e = -1.2 * ln(e + 1) for the Zipf-skewed many-expert layer;
* e_score_correction_bias ~ N(0, 0.01) in fp32 for the sigmoid layers;
* router gate weights W_g [E, H] ~ N(0, 1/H) (standard deviation H^-1/2, so
  the logits of N(0, 1) hidden rows are again about N(0, 1)), drawn in fp32
  and kept in fp32 or rounded to bf16 (MoEGate of the DeepSeek page holds the
  gate in the model dtype or, with router_fp32, in fp32).

No near-ties: a row of router logits whose routing decision is within
``delta`` of a tie (consecutive gaps among the K+1 best selection keys, and for
grouped routing the gap between the TG-th and (TG+1)-th group score) is
redrawn from the next draw of its stream.  The gap test evaluates the
selection keys in float64; it conditions the input distribution and is not
used by either implementation.

Decode-sized inputs are the first T rows of the matching prefill inputs.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

# Stream ids of the tensors; each tensor draws from its own seeded stream.
_LOGITS, _HIDDEN, _W13, _W2, _BIAS, _SW13, _SW2, _GATE = range(8)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    E: int
    K: int
    H: int
    I: int
    T: int
    act_dtype: str = "bf16"        # "f32" | "bf16"
    w_dtype: str = "bf16"          # "f32" | "bf16" | "fp8"
    scoring: str = "softmax"       # "softmax" | "sigmoid"
    renormalize: bool = True
    n_group: int = 0
    topk_group: int = 0
    rsf: float = 1.0
    logit_skew: str = "none"       # "none" | "zipf"
    correction_bias: bool = False
    shared: int = 0                # number of shared experts (0 or 1)
    shared_I: int = 0              # its intermediate size; 0 -> I
    seed: int = 0
    weight_seed: int = 0
    delta: float = 1e-3
    w_std: float = 0.02
    T_gen: int = 0                 # rows drawn (decode = first T rows); 0 -> T
    # activation variants (defaults: the plain SiLU-and-mul layer)
    non_gated: bool = False        # w13 [E, I, H], act = silu_a(x W1^T)
    swiglu_alpha: float = 0.0      # slope a of silu_a(z) = z sigmoid(a z); 0 -> 1
    swiglu_limit: float = 0.0      # clamp of gate (above) and up (both sides); 0 -> none
    weight_on_input: bool = False  # routing weight scales the expert input

    @property
    def fp8(self) -> bool:
        return self.w_dtype == "fp8"

    @property
    def Is(self) -> int:
        """Intermediate size of the shared expert."""
        return self.shared_I or self.I

    @property
    def rows_drawn(self) -> int:
        return max(self.T, self.T_gen)

    def with_T(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T, T_gen=max(self.T_gen, self.T))

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward: 6*T*K*H*I (+ 6*T*H*Is for a shared expert)."""
        return 6.0 * self.T * self.H * (self.K * self.I + self.shared * self.Is)


# The five layer configurations (sizes and distributions as stated above).
CONFIGS = {
    "tiny": MoEConfig("tiny", E=8, K=2, H=128, I=256, T=64, act_dtype="f32",
                      w_dtype="f32", seed=1, weight_seed=1, delta=1e-3),
    "mixtral": MoEConfig("mixtral", E=8, K=2, H=4096, I=14336, T=4096, seed=2,
                         weight_seed=2, delta=1e-3, T_gen=4096),
    "qwen": MoEConfig("qwen", E=128, K=8, H=2048, I=768, T=16384, seed=3,
                      weight_seed=3, logit_skew="zipf", delta=1e-3, T_gen=16384),
    "dsv3": MoEConfig("dsv3", E=256, K=8, H=7168, I=2048, T=8192, scoring="sigmoid",
                      n_group=8, topk_group=4, rsf=2.5, correction_bias=True,
                      seed=4, weight_seed=4, delta=1e-4, T_gen=8192),
    "dsv3_fp8": MoEConfig("dsv3_fp8", E=256, K=8, H=7168, I=2048, T=8192,
                          w_dtype="fp8", scoring="sigmoid", n_group=8, topk_group=4,
                          rsf=2.5, correction_bias=True, shared=1, seed=4,
                          weight_seed=5, delta=1e-4, T_gen=8192),
}
# Decode-sized variants: the first T rows of the prefill inputs.
CONFIGS["mixtral_decode"] = dataclasses.replace(CONFIGS["mixtral"], name="mixtral_decode", T=32)
CONFIGS["dsv3_decode"] = dataclasses.replace(CONFIGS["dsv3"], name="dsv3_decode", T=64)


def _rng(seed: int, stream: int, draw: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, stream, draw])


def _torch_seed(seed: int, stream: int, index: int) -> int:
    return (seed * 1_000_003 + stream * 10_007 + index) & 0x7FFF_FFFF_FFFF


def make_correction_bias(cfg: MoEConfig):
    """e_score_correction_bias ~ N(0, 0.01) in fp32, or None."""
    if not cfg.correction_bias:
        return None
    return (_rng(cfg.seed, _BIAS).standard_normal(cfg.E) * 0.01).astype(np.float32)


def _logit_skew(cfg: MoEConfig) -> np.ndarray:
    if cfg.logit_skew == "zipf":
        return -1.2 * np.log(np.arange(cfg.E, dtype=np.float64) + 1.0)
    return np.zeros(cfg.E)


def _rows_without_near_ties(cfg: MoEConfig, logits: np.ndarray, bias) -> np.ndarray:
    """True for rows whose routing decision is at least delta away from a tie."""
    l = logits.astype(np.float64)
    if cfg.scoring == "softmax":
        key = l
    else:
        key = 1.0 / (1.0 + np.exp(-l)) + (0.0 if bias is None else bias.astype(np.float64))
    T, E = key.shape
    ok = np.ones(T, dtype=bool)
    if cfg.n_group > 1:
        G, TG = cfg.n_group, cfg.topk_group
        per = E // G
        grouped = np.sort(key.reshape(T, G, per), axis=2)[:, :, ::-1]
        if bias is not None and per >= 2:
            gscore = grouped[:, :, 0] + grouped[:, :, 1]
        else:
            gscore = grouped[:, :, 0]
        order = np.argsort(-gscore, axis=1, kind="stable")
        gs = np.take_along_axis(gscore, order, axis=1)
        if TG < G:
            ok &= (gs[:, TG - 1] - gs[:, TG]) >= cfg.delta
        keep = np.zeros((T, G), dtype=bool)
        np.put_along_axis(keep, order[:, :TG], True, axis=1)
        key = np.where(np.repeat(keep, per, axis=1), key, -np.inf)
    top = -np.sort(-key, axis=1)[:, : cfg.K + 1]
    top = top[:, : min(cfg.K + 1, top.shape[1])]
    finite = np.isfinite(top)
    gaps = top[:, :-1] - top[:, 1:]
    gap_ok = np.where(finite[:, 1:], gaps >= cfg.delta, True)
    ok &= gap_ok.all(axis=1)
    return ok


def make_logits(cfg: MoEConfig, T: int | None = None) -> np.ndarray:
    """Router logits [T, E] fp32 with no near-ties (first T rows of the drawn rows)."""
    T = cfg.T if T is None else T
    rows = max(T, cfg.rows_drawn)
    bias = make_correction_bias(cfg)
    skew = _logit_skew(cfg)
    logits = (_rng(cfg.seed, _LOGITS, 0).standard_normal((rows, cfg.E)) + skew).astype(np.float32)
    bad = ~_rows_without_near_ties(cfg, logits, bias)
    draw = 1
    while bad.any():
        if draw > 10_000:
            raise RuntimeError("could not draw router logits without near-ties")
        fresh = (_rng(cfg.seed, _LOGITS, draw).standard_normal((rows, cfg.E)) + skew).astype(np.float32)
        idx = np.nonzero(bad)[0]
        logits[idx] = fresh[idx]
        bad[idx] = ~_rows_without_near_ties(cfg, logits[idx], bias)
        draw += 1
    return np.ascontiguousarray(logits[:T])


def _act_torch_dtype(cfg: MoEConfig):
    return torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16


def make_hidden(cfg: MoEConfig, T: int | None = None, device="cpu") -> torch.Tensor:
    """hidden [T, H] ~ N(0,1) in the activation dtype (first T of the drawn rows)."""
    T = cfg.T if T is None else T
    rows = max(T, cfg.rows_drawn)
    g = torch.Generator(device="cpu")
    g.manual_seed(_torch_seed(cfg.seed, _HIDDEN, 0))
    x = torch.randn(rows, cfg.H, generator=g, dtype=torch.float32)[:T]
    return x.to(_act_torch_dtype(cfg)).contiguous().to(device)


def _block_quant_e4m3(w: torch.Tensor):
    """[N, K] fp32 -> (codes uint8 [N, K], scales fp32 [N/128, K/128])."""
    N, K = w.shape
    blocks = w.reshape(N // 128, 128, K // 128, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.clamp(amax, min=1e-10) / 448.0
    q = (blocks / scale[:, None, :, None]).clamp(-448.0, 448.0).reshape(N, K)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32).contiguous()


def _draw_matrix(seed: int, stream: int, index: int, shape, std: float, device):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, stream, index))
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def _store_weights(cfg, count, stream, shape, device):
    """Draw `count` matrices of `shape` and store them in the weight dtype."""
    N, K = shape
    if cfg.w_dtype == "fp8":
        codes = torch.empty(count, N, K, dtype=torch.uint8, device=device)
        scales = torch.empty(count, N // 128, K // 128, dtype=torch.float32, device=device)
    else:
        dt = torch.float32 if cfg.w_dtype == "f32" else torch.bfloat16
        codes = torch.empty(count, N, K, dtype=dt, device=device)
        scales = None
    for e in range(count):
        w = _draw_matrix(cfg.weight_seed, stream, e, shape, cfg.w_std, device)
        if scales is not None:
            codes[e], scales[e] = _block_quant_e4m3(w)
        else:
            codes[e] = w.to(codes.dtype)
        del w
    return codes, scales


def make_weights(cfg: MoEConfig, device="cpu") -> dict:
    """Expert weights: w13 [E, 2I, H] (gate rows first, then up rows) and
    w2 [E, H, I]; fp8 layers also get the 128x128 block scales and, with a
    shared expert, shared_w13 [2Is, H] / shared_w2 [H, Is] in the same
    format."""
    out = {}
    n13 = cfg.I if cfg.non_gated else 2 * cfg.I
    out["w13"], out["w13_scale"] = _store_weights(cfg, cfg.E, _W13, (n13, cfg.H), device)
    out["w2"], out["w2_scale"] = _store_weights(cfg, cfg.E, _W2, (cfg.H, cfg.I), device)
    if cfg.shared:
        s13 = cfg.Is if cfg.non_gated else 2 * cfg.Is
        a, sa = _store_weights(cfg, 1, _SW13, (s13, cfg.H), device)
        b, sb = _store_weights(cfg, 1, _SW2, (cfg.H, cfg.Is), device)
        out["shared_w13"], out["shared_w2"] = a[0], b[0]
        out["shared_w13_scale"] = None if sa is None else sa[0]
        out["shared_w2_scale"] = None if sb is None else sb[0]
    return out


def make_gate(cfg: MoEConfig, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """Router gate weights [E, H] ~ N(0, 1/H) in fp32 ("f32") or bf16."""
    w = _draw_matrix(cfg.weight_seed, _GATE, 0, (cfg.E, cfg.H), cfg.H ** -0.5, "cpu")
    return w.to(torch.float32 if dtype == "f32" else torch.bfloat16).contiguous().to(device)


def make_inputs(cfg: MoEConfig, T: int | None = None, device="cpu", weight_device=None) -> dict:
    """All inputs of one forward as torch tensors on `device`."""
    T = cfg.T if T is None else T
    wdev = device if weight_device is None else weight_device
    d = {
        "hidden": make_hidden(cfg, T, device),
        "router_logits": torch.from_numpy(make_logits(cfg, T)).to(device),
    }
    b = make_correction_bias(cfg)
    d["e_score_correction_bias"] = None if b is None else torch.from_numpy(b).to(device)
    d.update(make_weights(cfg, wdev))
    return d


def tensor_bits(t: torch.Tensor | None) -> np.ndarray | None:
    """Host numpy view of a tensor's raw values (bf16 as uint16, fp8 as uint8)."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    return t.numpy()
